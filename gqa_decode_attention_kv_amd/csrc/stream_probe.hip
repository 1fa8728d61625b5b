// Measurement probes, not part of the decode path: a plain streaming read of
// device memory, used to find the HBM read rate this part sustains in
// practice, the ceiling the bandwidth-bound decode kernels are compared with.
//
// Each work-group of four waves reads one contiguous range (one sequential
// stream per work-group) with 16-byte non-temporal loads, eight in flight
// per lane.  The loaded words are folded into a value that is stored only
// if it equals a constant no input here produces, so the loads stay live
// and almost nothing is written.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n,
                                                               size_t per_group, uint32_t* sink) {
  const size_t begin = static_cast<size_t>(blockIdx.x) * per_group;
  const size_t end = begin + per_group < n ? begin + per_group : n;
  uint32_t acc = 0;
  size_t i = begin + threadIdx.x;
  for (; i + (kInFlight - 1) * kThreads < end; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(src + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < end; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

// The same read over pieces of 2^lcpp 16-byte chunks scattered through the
// buffer: work-group g reads pieces order[g * per_group ..] in turn, the
// access pattern of a paged cache (one piece = one cache block of one kv
// head).  Chunk i of the group's range is chunk i % 2^lcpp of its piece
// i / 2^lcpp.  The group's piece indices are staged in LDS before the first
// load, so no load waits on a lookup in global memory (a paged kernel reads
// its block ids ahead of its cache loads in the same way).
constexpr int kMaxGroupPieces = 4096;

__global__ __launch_bounds__(kThreads) void gather_read_kernel(const u32x4* __restrict__ src, int lcpp,
                                                               const int* __restrict__ order, int n_pieces,
                                                               int pieces_in_src, int per_group, uint32_t* sink) {
  __shared__ int piece_of[kMaxGroupPieces];
  const int p0 = blockIdx.x * per_group;
  const int p1 = p0 + per_group < n_pieces ? p0 + per_group : n_pieces;
  for (int k = threadIdx.x; k < p1 - p0; k += kThreads) piece_of[k] = min(max(order[p0 + k], 0), pieces_in_src - 1);
  __syncthreads();
  const int end = (p1 - p0) << lcpp;
  auto addr = [&](int i) {
    return (static_cast<int64_t>(piece_of[i >> lcpp]) << lcpp) + (i & ((1 << lcpp) - 1));
  };
  uint32_t acc = 0;
  int i = threadIdx.x;
  for (; i + (kInFlight - 1) * kThreads < end; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = __builtin_nontemporal_load(src + addr(i + k * kThreads));
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < end; i += kThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + addr(i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` bytes at `src` (device, 16-byte aligned, a multiple of 16),
// `bytes_per_group` bytes per work-group (a multiple of 16).  `sink` is a
// device buffer of at least ceil(bytes / bytes_per_group) words that is
// practically never written.  Returns 0, or a HIP error code (nothing is
// launched when the arguments are refused: 1 = invalid argument).
extern "C" int uaii_probe_stream_read(const void* src, size_t bytes, size_t bytes_per_group,
                                      uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 || bytes_per_group == 0 ||
      bytes_per_group % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return 1;
  const size_t n = bytes / 16;
  const size_t per = bytes_per_group / 16;
  const size_t groups = (n + per - 1) / per;
  if (groups > 0x7FFFFFFFu) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), n, per, sink);
  return static_cast<int>(hipGetLastError());
}

// Reads n_pieces pieces of piece_bytes bytes (16 times a power of two) of `src`
// (device, 16-byte aligned, pieces_in_src * piece_bytes bytes readable),
// piece k starting at byte order[k] * piece_bytes; `order` is a device
// array of n_pieces indices (clamped to [0, pieces_in_src) on the device).
// pieces_per_group pieces per work-group (at most 4096); `sink` as for
// uaii_probe_stream_read, of at least ceil(n_pieces / pieces_per_group)
// words.  Returns 0, or a HIP error code (1 = invalid argument, nothing
// launched).
extern "C" int uaii_probe_gather_read(const void* src, size_t pieces_in_src, size_t piece_bytes, const int* order,
                                      int n_pieces, int pieces_per_group, uint32_t* sink, void* stream) {
  if (src == nullptr || order == nullptr || sink == nullptr || piece_bytes < 16 || piece_bytes % 16 != 0 ||
      n_pieces <= 0 || pieces_per_group <= 0 || pieces_per_group > kMaxGroupPieces || pieces_in_src == 0 ||
      pieces_in_src > 0x7FFFFFFF ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return 1;
  const size_t cpp = piece_bytes / 16;
  if ((cpp & (cpp - 1)) != 0 || cpp > (size_t{1} << 20)) return 1;
  int lcpp = 0;
  while ((size_t{1} << lcpp) < cpp) ++lcpp;
  // The group's chunk index must fit an int.
  if ((static_cast<int64_t>(pieces_per_group) << lcpp) > 0x7FFFFFFF) return 1;
  const int groups = (n_pieces + pieces_per_group - 1) / pieces_per_group;
  hipLaunchKernelGGL(gather_read_kernel, dim3(static_cast<unsigned>(groups)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     lcpp, order, n_pieces, static_cast<int>(pieces_in_src),
                     pieces_per_group, sink);
  return static_cast<int>(hipGetLastError());
}

// Stable compaction of the kept tokens (TokenGate article, section "How does
// TokenGate learned token pruning work?": layers above the gate process only
// the kept tokens and create no KV entries for pruned ones; section "What is
// token-gated attention?": each kept token's score becomes its logit bias).
//
// Kept token t goes to row r = number of kept tokens before t, so rows follow
// the original order prompt by prompt.  Three kernels:
//   cmp_count   per chunk of kCmpChunk tokens: number of kept flags
//   cmp_scan    one workgroup: exclusive prefix over the chunk counts
//   cmp_gather  per chunk: block scan of the flags gives each kept token its
//               row; positions, biases and indices are written by the
//               owning thread, hidden rows are copied by whole waves in
//               16-byte units (a byte-exact copy).
#include "tg_common.h"

namespace tg {
namespace {

constexpr int kCmpChunk = 1024;   // tokens per chunk
constexpr int kCmpThreads = 256;  // 4 tokens per thread

__global__ __launch_bounds__(kCmpThreads) void cmp_count(const uint8_t* __restrict__ keep,
                                                         int64_t T, int* __restrict__ counts) {
  const int64_t base = (int64_t)blockIdx.x * kCmpChunk + threadIdx.x * 4;
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (base + j < T) c += keep[base + j] ? 1 : 0;
  __shared__ int wsum[kCmpThreads / 64];
  int v = c;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kCmpThreads / 64; ++w) s += wsum[w];
    counts[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(1024) void cmp_scan(const int* __restrict__ counts, int n,
                                                 int* __restrict__ offsets) {
  // Sequential rounds of 1024 with a carry; inside a round, a Hillis-Steele
  // scan in LDS (integer, exact).
  __shared__ int buf[1024];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int x = (i < n) ? counts[i] : 0;
    buf[threadIdx.x] = x;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int y = (threadIdx.x >= (unsigned)off) ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += y;
      __syncthreads();
    }
    if (i < n) offsets[i] = carry + buf[threadIdx.x] - x;
    __syncthreads();
    if (threadIdx.x == 1023) carry += buf[1023];
    __syncthreads();
  }
}

__device__ __forceinline__ int find_prompt_c(const int32_t* cu, int B, int64_t t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kCmpThreads) void cmp_gather(
    const char* __restrict__ hidden, int64_t ld_bytes, int row_bytes, int vec16,
    const int32_t* __restrict__ pos, const float* __restrict__ scores,
    const uint8_t* __restrict__ keep, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ db, const int32_t* __restrict__ de, int B, int64_t T,
    const int* __restrict__ offsets, int64_t Kt, char* __restrict__ hidden_out,
    int32_t* __restrict__ pos_out, float* __restrict__ bias_out,
    int32_t* __restrict__ kept_idx_out) {
  __shared__ int wsum[kCmpThreads / 64];
  __shared__ int list_t[kCmpChunk];
  __shared__ int list_r[kCmpChunk];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * kCmpChunk + tid * 4;
  int f[4];
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = (base + j < T && keep[base + j]) ? 1 : 0;
    c += f[j];
  }
  // exclusive prefix of c over the workgroup: wave inclusive scan + wave sums
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0, total = 0;
  for (int w = 0; w < kCmpThreads / 64; ++w) {
    if (w < wave) wbase += wsum[w];
    total += wsum[w];
  }
  int local = wbase + incl - c;
  const int row0 = offsets[blockIdx.x];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!f[j]) continue;
    const int64_t t = base + j;
    const int r = row0 + local;
    if (r < Kt) {  // flags beyond the stated Kt write nothing
      const int b = find_prompt_c(cu, B, t);
      const int64_t rel = t - cu[b];
      const bool in_doc = rel >= db[b] && rel < de[b];
      pos_out[r] = pos ? pos[t] : (int32_t)rel;
      bias_out[r] = in_doc ? scores[t] : 0.0f;
      if (kept_idx_out) kept_idx_out[r] = (int32_t)t;
    }
    list_t[local] = (int)(t - (int64_t)blockIdx.x * kCmpChunk);
    list_r[local] = r < Kt ? r : -1;
    ++local;
  }
  __syncthreads();
  // Row copies: wave w takes list entries w, w + 4, ...
  const int64_t chunk0 = (int64_t)blockIdx.x * kCmpChunk;
  for (int e = wave; e < total; e += kCmpThreads / 64) {
    if (list_r[e] < 0) continue;
    const char* src = hidden + (chunk0 + list_t[e]) * ld_bytes;
    char* dst = hidden_out + (int64_t)list_r[e] * row_bytes;
    if (vec16 == 1) {
      const int n16 = row_bytes >> 4;
      for (int u = lane; u < n16; u += 64)
        reinterpret_cast<uint4*>(dst)[u] = reinterpret_cast<const uint4*>(src)[u];
    } else if (vec16 == 0) {  // element-wise copy, 4-byte elements
      for (int u = lane; u < (row_bytes >> 2); u += 64)
        reinterpret_cast<uint32_t*>(dst)[u] = reinterpret_cast<const uint32_t*>(src)[u];
    } else {  // element-wise copy, 2-byte elements
      for (int u = lane; u < (row_bytes >> 1); u += 64)
        reinterpret_cast<uint16_t*>(dst)[u] = reinterpret_cast<const uint16_t*>(src)[u];
    }
  }
}

}  // namespace

size_t compact_workspace_bytes(int /*B*/, int64_t T) {
  const size_t n = (size_t)((T + kCmpChunk - 1) / kCmpChunk) + 1;
  return 2 * n * sizeof(int);
}

hipError_t launch_compact(const void* hidden, int64_t ld, int D, int elem_bytes, const int32_t* pos,
                          const float* scores, const uint8_t* keep, const int32_t* cu,
                          const int32_t* db, const int32_t* de, int B, int64_t T, int64_t Kt,
                          void* hidden_out, int32_t* pos_out, float* bias_out,
                          int32_t* kept_idx_out, void* ws, hipStream_t s) {
  if (T == 0 || B == 0) return hipSuccess;
  const int nchunks = (int)((T + kCmpChunk - 1) / kCmpChunk);
  int* counts = static_cast<int*>(ws);
  int* offsets = counts + nchunks + 1;
  const int row_bytes = D * elem_bytes;
  const int64_t ld_bytes = ld * elem_bytes;
  // copy mode: 1 = 16-byte units, 0 = 4-byte elements, 2 = 2-byte elements
  int vec16 = elem_bytes == 4 ? 0 : 2;
  if ((row_bytes % 16) == 0 && (ld_bytes % 16) == 0 && ((uintptr_t)hidden % 16) == 0 &&
      ((uintptr_t)hidden_out % 16) == 0)
    vec16 = 1;
  hipLaunchKernelGGL(cmp_count, dim3(nchunks), dim3(kCmpThreads), 0, s, keep, T, counts);
  hipLaunchKernelGGL(cmp_scan, dim3(1), dim3(1024), 0, s, counts, nchunks, offsets);
  hipLaunchKernelGGL(cmp_gather, dim3(nchunks), dim3(kCmpThreads), 0, s,
                     static_cast<const char*>(hidden), ld_bytes, row_bytes, vec16, pos, scores,
                     keep, cu, db, de, B, T, offsets, Kt, static_cast<char*>(hidden_out), pos_out,
                     bias_out, kept_idx_out);
  return hipGetLastError();
}

}  // namespace tg

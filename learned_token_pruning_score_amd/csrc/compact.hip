// Stable compaction of the kept tokens (TokenGate article, section "How does
// TokenGate learned token pruning work?": layers above the gate process only
// the kept tokens and create no KV entries for pruned ones; section "What is
// token-gated attention?": each kept token's score becomes its logit bias).
//
// Kept token t goes to row r = number of kept tokens before t, so rows follow
// the original order prompt by prompt.  Kernels:
//   cmp_count  per chunk of kCmpChunk tokens: number of kept flags
//   cmp_index  per chunk: its base row is the sum of the counts before it;
//              a block scan of the flags gives each kept token its row, and
//              the owning thread writes the row's source token
//   (up to kFuseMaxT tokens one kernel, cmp_index_fused, does both: each
//   workgroup counts the flags before its chunk itself)
//   cmp_copy   one wave per kept row: the hidden row is copied byte-exactly
//              in 16-byte units (or element by element when rows or
//              pointers are not 16-byte aligned), every lane issuing all its
//              loads before its stores; lane 0 writes the row's position,
//              bias and source index
// Integer arithmetic only; deterministic.
#include "tg_common.h"

namespace tg {
namespace {

constexpr int kCmpChunk = 1024;   // tokens per chunk
constexpr int kCmpThreads = 256;  // 4 tokens per thread
constexpr int kRowsPerCopyWG = 4;  // one wave per row

__global__ __launch_bounds__(kCmpThreads) void cmp_count(const uint8_t* __restrict__ keep,
                                                         int64_t T, int* __restrict__ counts) {
  const int64_t base = (int64_t)blockIdx.x * kCmpChunk + threadIdx.x * 4;
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (base + j < T) c += keep[base + j] ? 1 : 0;
  __shared__ int wsum[kCmpThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kCmpThreads / 64; ++w) s += wsum[w];
    counts[blockIdx.x] = s;
  }
}

__device__ __forceinline__ int find_prompt_c(const int32_t* cu, int B, int64_t t) {
  int lo = 0, hi = B - 1;  // largest b with cu[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kCmpThreads) void cmp_index(
    const uint8_t* __restrict__ keep, int64_t T, const int* __restrict__ counts, int64_t Kt,
    int32_t* __restrict__ src_out) {
  __shared__ int wsum[kCmpThreads / 64];
  __shared__ int s_row0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // base row: sum of the counts of all earlier chunks (fixed order)
  int pre = 0;
  for (int i = tid; i < (int)blockIdx.x; i += kCmpThreads) pre += counts[i];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pre += __shfl_xor(pre, off);
  if (lane == 0) wsum[wave] = pre;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kCmpThreads / 64; ++w) s += wsum[w];
    s_row0 = s;
  }
  __syncthreads();
  const int row0 = s_row0;
  __syncthreads();  // wsum is reused below

  const int64_t base = (int64_t)blockIdx.x * kCmpChunk + tid * 4;
  int f[4];
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = (base + j < T && keep[base + j]) ? 1 : 0;
    c += f[j];
  }
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += wsum[w];
  int r = row0 + wbase + incl - c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!f[j]) continue;
    if (r < Kt) src_out[r] = (int32_t)(base + j);  // flags beyond the stated Kt write nothing
    ++r;
  }
}

// Count and index in one kernel, for inputs of up to kFuseMaxT tokens: each
// workgroup counts the kept flags before its chunk of kFuseChunk tokens
// itself (16 flags per 16-byte load, every load of a thread in flight at
// once), instead of summing per-chunk counts written by an earlier kernel.
// The flag array must be 16-byte aligned (checked on the host).
constexpr int kFuseThreads = 1024;
constexpr int kFuseChunk = 4 * kFuseThreads;
constexpr int64_t kFuseMaxT = (int64_t)1 << 18;
constexpr int kFuseLoads = (int)(kFuseMaxT / 16 / kFuseThreads);  // 16-byte loads per thread at most

// nonzero bytes of a 32-bit word (a flag is kept when nonzero)
__device__ __forceinline__ int nz_bytes(unsigned w) {
  return __popc((((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u);
}

__global__ __launch_bounds__(kFuseThreads) void cmp_index_fused(
    const uint8_t* __restrict__ keep, int64_t T, int64_t Kt, int32_t* __restrict__ src_out) {
  __shared__ int wsum[kFuseThreads / 64];
  __shared__ int s_row0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kFuseChunk;
  // kept flags before the chunk (c0 / 16 whole 16-byte words)
  const uint4* k4 = reinterpret_cast<const uint4*>(keep);
  const int n16 = (int)(c0 / 16);
  uint4 w[kFuseLoads];
#pragma unroll
  for (int j = 0; j < kFuseLoads; ++j) {
    const int i = tid + j * kFuseThreads;
    w[j] = i < n16 ? k4[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  int pre = 0;
#pragma unroll
  for (int j = 0; j < kFuseLoads; ++j) pre += nz_bytes(w[j].x) + nz_bytes(w[j].y) + nz_bytes(w[j].z) + nz_bytes(w[j].w);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pre += __shfl_xor(pre, off);
  if (lane == 0) wsum[wave] = pre;
  __syncthreads();
  if (tid == 0) {
    int sum = 0;
    for (int v = 0; v < kFuseThreads / 64; ++v) sum += wsum[v];
    s_row0 = sum;
  }
  __syncthreads();
  const int row0 = s_row0;
  __syncthreads();  // wsum is reused below

  const int64_t base = c0 + tid * 4;
  int f[4];
  int c = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = (base + j < T && keep[base + j]) ? 1 : 0;
    c += f[j];
  }
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0;
  for (int v = 0; v < wave; ++v) wbase += wsum[v];
  int r = row0 + wbase + incl - c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!f[j]) continue;
    if (r < Kt) src_out[r] = (int32_t)(base + j);  // flags beyond the stated Kt write nothing
    ++r;
  }
}

// MODE 1: 16-byte units; 0: 4-byte elements; 2: 2-byte elements.
template <int MODE>
__global__ __launch_bounds__(64 * kRowsPerCopyWG) void cmp_copy(
    const char* __restrict__ hidden, int64_t ld_bytes, int row_bytes,
    const int32_t* __restrict__ src, int64_t T, int64_t Kt, char* __restrict__ hidden_out,
    const int32_t* __restrict__ pos, const float* __restrict__ scores,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ db,
    const int32_t* __restrict__ de, int B, int32_t* __restrict__ pos_out,
    float* __restrict__ bias_out, int32_t* __restrict__ kept_idx_out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerCopyWG + (threadIdx.x >> 6);
  if (r >= Kt) return;
  // clamped: with fewer kept flags than Kt (a caller error) the unwritten
  // rows copy some valid row instead of reading outside `hidden`
  const int64_t t = min(max((int64_t)src[r], (int64_t)0), T - 1);
  // the row's position, bias and source index, written after the copy so
  // that their loads do not hold the copy's back
  auto meta = [&]() __attribute__((always_inline)) {
    if (lane != 0) return;
    const int b = find_prompt_c(cu, B, t);
    const int64_t rel = t - cu[b];
    const bool in_doc = rel >= db[b] && rel < de[b];
    pos_out[r] = pos ? pos[t] : (int32_t)rel;
    bias_out[r] = in_doc ? scores[t] : 0.0f;
    if (kept_idx_out) kept_idx_out[r] = (int32_t)t;
  };
  const char* s = hidden + t * ld_bytes;
  char* d = hidden_out + r * row_bytes;
  if (MODE == 1) {
    const int n16 = row_bytes >> 4;
    const uint4* s4 = reinterpret_cast<const uint4*>(s);
    uint4* d4 = reinterpret_cast<uint4*>(d);
    int u = lane;
    for (; u + 192 < n16; u += 256) {  // four loads in flight per lane
      const uint4 a = s4[u], b = s4[u + 64], c = s4[u + 128], e = s4[u + 192];
      d4[u] = a;
      d4[u + 64] = b;
      d4[u + 128] = c;
      d4[u + 192] = e;
    }
    for (; u < n16; u += 64) d4[u] = s4[u];
  } else if (MODE == 0) {
    for (int u = lane; u < (row_bytes >> 2); u += 64)
      reinterpret_cast<uint32_t*>(d)[u] = reinterpret_cast<const uint32_t*>(s)[u];
  } else {
    for (int u = lane; u < (row_bytes >> 1); u += 64)
      reinterpret_cast<uint16_t*>(d)[u] = reinterpret_cast<const uint16_t*>(s)[u];
  }
  meta();
}

}  // namespace

size_t compact_workspace_bytes(int /*B*/, int64_t T) {
  const size_t n = (size_t)((T + kCmpChunk - 1) / kCmpChunk) + 1;
  const size_t counts = (n * sizeof(int) + 255) & ~(size_t)255;
  return counts + (size_t)T * sizeof(int32_t);  // chunk counts + row source index
}

hipError_t launch_compact(const void* hidden, int64_t ld, int D, int elem_bytes, const int32_t* pos,
                          const float* scores, const uint8_t* keep, const int32_t* cu,
                          const int32_t* db, const int32_t* de, int B, int64_t T, int64_t Kt,
                          void* hidden_out, int32_t* pos_out, float* bias_out,
                          int32_t* kept_idx_out, void* ws, hipStream_t s) {
  if (T == 0 || B == 0) return hipSuccess;
  const int nchunks = (int)((T + kCmpChunk - 1) / kCmpChunk);
  int* counts = static_cast<int*>(ws);
  const size_t counts_bytes = (((size_t)nchunks + 1) * sizeof(int) + 255) & ~(size_t)255;
  int32_t* src = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + counts_bytes);
  const int row_bytes = D * elem_bytes;
  const int64_t ld_bytes = ld * elem_bytes;
  if (T <= kFuseMaxT && ((uintptr_t)keep % 16) == 0) {
    hipLaunchKernelGGL(cmp_index_fused, dim3((unsigned)((T + kFuseChunk - 1) / kFuseChunk)), dim3(kFuseThreads),
                       0, s, keep, T, Kt, src);
  } else {
    hipLaunchKernelGGL(cmp_count, dim3(nchunks), dim3(kCmpThreads), 0, s, keep, T, counts);
    hipLaunchKernelGGL(cmp_index, dim3(nchunks), dim3(kCmpThreads), 0, s, keep, T, counts, Kt, src);
  }
  if (Kt > 0) {
    const dim3 grid((unsigned)((Kt + kRowsPerCopyWG - 1) / kRowsPerCopyWG));
    const dim3 block(64 * kRowsPerCopyWG);
    const auto* h = static_cast<const char*>(hidden);
    auto* o = static_cast<char*>(hidden_out);
    if ((row_bytes % 16) == 0 && (ld_bytes % 16) == 0 && ((uintptr_t)hidden % 16) == 0 &&
        ((uintptr_t)hidden_out % 16) == 0)
      hipLaunchKernelGGL(cmp_copy<1>, grid, block, 0, s, h, ld_bytes, row_bytes, src, T, Kt, o, pos,
                         scores, cu, db, de, B, pos_out, bias_out, kept_idx_out);
    else if (elem_bytes == 4)
      hipLaunchKernelGGL(cmp_copy<0>, grid, block, 0, s, h, ld_bytes, row_bytes, src, T, Kt, o, pos,
                         scores, cu, db, de, B, pos_out, bias_out, kept_idx_out);
    else
      hipLaunchKernelGGL(cmp_copy<2>, grid, block, 0, s, h, ld_bytes, row_bytes, src, T, Kt, o, pos,
                         scores, cu, db, de, B, pos_out, bias_out, kept_idx_out);
  }
  return hipGetLastError();
}

}  // namespace tg

// Document-only top-K selection (TokenGate article, section "How does
// TokenGate learned token pruning work?": a top-K selector keeps the
// highest-scoring tokens, only the document is prunable, the question never
// is).
//
// Order: score descending, then token index ascending.  Scores map to 32-bit
// keys whose unsigned order is that score order (-0.0 folded onto +0.0, every
// NaN onto key 0, below -inf).  Per prompt, an MSB-first radix select over
// three digits (11, 11, 10 bits) finds theta, the key of the k-th best
// document token, and how many tokens of key theta must be kept; a tie pass
// turns that count into an index bound only when some equal keys must be
// dropped.  A token is kept when it lies outside the document, or its key is
// above theta, or its key equals theta and its index is at most the bound.
//
// Kernels (all on the caller's stream, no host sync):
//   sel_init   per prompt: state from (doc span, budget); clears histogram
//   sel_hist   per (chunk, prompt): LDS histogram of the current digit over
//              keys matching the chosen prefix, flushed with integer atomics
//   sel_pick   per prompt: suffix scan of the histogram picks the digit;
//              after the last digit, the index bound among keys equal to
//              theta when not all of them are kept
//   sel_mark   per token: keep flag
// Integer atomics only: the histogram, and so every result, is independent
// of execution order.
#include <limits.h>

#include "tg_common.h"

namespace tg {
namespace {

constexpr int kBins = 2048;
constexpr int kHistChunk = 4096;  // keys per sel_hist workgroup
constexpr int kHistThreads = 256;

struct SelState {
  int lo, hi;          // global doc span [lo, hi)
  int k_rem;           // keys still to place at/below the current prefix
  int active;          // 1 while the radix passes must run
  int mode;            // 0: keep no document token, 1: keep all, 2: radix
  unsigned prefix;     // chosen high bits of theta
  unsigned mask;       // which bits of prefix are fixed
  unsigned theta;      // final threshold key
  int idx_bound;       // keep key == theta iff index <= idx_bound
  int n_eq;            // number of keys equal to theta
  int pad[6];
};
static_assert(sizeof(SelState) == 64, "state size");

__device__ __forceinline__ unsigned score_key(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                     // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Digit p: bits [shift, shift + width).
__device__ __forceinline__ int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__device__ __forceinline__ unsigned digit_mask(int p) { return p == 2 ? 0x3ffu : 0x7ffu; }

__global__ __launch_bounds__(256) void sel_init(SelState* st, unsigned* hist,
                                                const int32_t* cu, const int32_t* db,
                                                const int32_t* de, const int32_t* budget) {
  const int b = blockIdx.x;
  unsigned* h = hist + (size_t)b * kBins;
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) h[i] = 0u;
  if (threadIdx.x == 0) {
    SelState s;
    s.lo = cu[b] + db[b];
    s.hi = cu[b] + de[b];
    const int n = s.hi - s.lo;
    const int k = min(budget[b], n);
    s.k_rem = k;
    s.prefix = 0u;
    s.mask = 0u;
    s.n_eq = 0;
    if (k <= 0) {            // keep no document token
      s.active = 0;
      s.mode = 0;
      s.theta = 0xffffffffu;  // above every key
      s.idx_bound = -1;
    } else if (k >= n) {     // keep the whole document
      s.active = 0;
      s.mode = 1;
      s.theta = 0u;
      s.idx_bound = INT_MAX;
    } else {
      s.active = 1;
      s.mode = 2;
      s.theta = 0u;
      s.idx_bound = INT_MAX;
    }
    for (int i = 0; i < 6; ++i) s.pad[i] = 0;
    st[b] = s;
  }
}

__global__ __launch_bounds__(kHistThreads) void sel_hist(const float* __restrict__ scores,
                                                         const SelState* st, unsigned* hist,
                                                         int pass) {
  const int b = blockIdx.y;
  const SelState s = st[b];
  if (!s.active) return;
  const int64_t c0 = (int64_t)s.lo + (int64_t)blockIdx.x * kHistChunk;
  if (c0 >= s.hi) return;
  const int64_t c1 = min((int64_t)s.hi, c0 + kHistChunk);

  __shared__ unsigned lh[kBins];
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) lh[i] = 0u;
  __syncthreads();
  const int sh = digit_shift(pass);
  const unsigned dm = digit_mask(pass);
  for (int64_t t = c0 + threadIdx.x; t < c1; t += kHistThreads) {
    const unsigned key = score_key(scores[t]);
    if ((key & s.mask) == s.prefix) atomicAdd(&lh[(key >> sh) & dm], 1u);
  }
  __syncthreads();
  unsigned* gh = hist + (size_t)b * kBins;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) {
    const unsigned c = lh[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// One workgroup of 1024 threads per prompt; thread i owns bins 2i, 2i + 1.
// The digit is the bin where the count of keys in higher bins first reaches
// k_rem; the counts above each thread come from an exclusive scan run from
// the top bin down (wave shuffles, then the 16 wave totals).  The histogram
// is cleared for the next pass.  After the last digit, theta is exact; if
// fewer than all keys equal to theta are kept, the same workgroup walks the
// document in index order to find the index bound (1024 tokens per round,
// stopping at the round that holds the k_rem-th equal key).
__global__ __launch_bounds__(1024) void sel_pick(const float* __restrict__ scores, SelState* st,
                                                 unsigned* hist, int pass) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ SelState s;
  __shared__ unsigned wtot[16];
  __shared__ int s_digit;
  __shared__ unsigned s_above, s_bin;
  if (tid == 0) {
    s = st[b];
    s_digit = 0;
    s_above = 0u;
    s_bin = 0u;
  }
  __syncthreads();
  if (!s.active) return;
  unsigned* h = hist + (size_t)b * kBins;
  // thread j (counted from the top) owns bins hi = 2047 - 2j and hi - 1
  const int hi_bin = kBins - 1 - 2 * tid;
  const unsigned c_hi = h[hi_bin], c_lo = h[hi_bin - 1];
  h[hi_bin] = 0u;
  h[hi_bin - 1] = 0u;
  const unsigned mine = c_hi + c_lo;
  unsigned incl = mine;  // inclusive scan over threads, top bins first
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  unsigned above = incl - mine;
  for (int w = 0; w < wave; ++w) above += wtot[w];
  const unsigned k_rem = (unsigned)s.k_rem;
  if (above < k_rem && k_rem <= above + mine) {
    if (above + c_hi >= k_rem) {
      s_digit = hi_bin;
      s_above = above;
      s_bin = c_hi;
    } else {
      s_digit = hi_bin - 1;
      s_above = above + c_hi;
      s_bin = c_lo;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int sh = digit_shift(pass);
    s.prefix |= (unsigned)s_digit << sh;
    s.mask |= digit_mask(pass) << sh;
    s.k_rem -= (int)s_above;
    if (pass == 2) {  // every bit fixed: theta found
      s.theta = s.prefix;
      s.active = 0;
      s.n_eq = (int)s_bin;  // keys equal to theta
    }
  }
  __syncthreads();
  if (pass == 2 && s.k_rem < s.n_eq) {
    // keep only the first k_rem keys equal to theta, by index
    int seen = 0;
    for (int base = s.lo; base < s.hi; base += 1024) {
      const int t = base + tid;
      const int eq = (t < s.hi) && (score_key(scores[t]) == s.theta);
      const unsigned long long bal = __ballot(eq);
      const int in_wave = __popcll(bal & ((lane == 63) ? ~0ull : ((2ull << lane) - 1)));
      __syncthreads();
      if (lane == 63) wtot[wave] = (unsigned)in_wave;
      __syncthreads();
      int before = 0, round_total = 0;
      for (int w = 0; w < 16; ++w) {
        if (w < wave) before += (int)wtot[w];
        round_total += (int)wtot[w];
      }
      if (eq && seen + before + in_wave == s.k_rem) s.idx_bound = t;
      seen += round_total;
      if (seen >= s.k_rem) break;
    }
  }
  __syncthreads();
  if (tid == 0) st[b] = s;
}

__device__ __forceinline__ int find_prompt(const int32_t* cu, int B, int64_t t) {
  int lo = 0, hi = B - 1;  // largest b with cu[b] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void sel_mark(const float* __restrict__ scores,
                                                const SelState* __restrict__ st,
                                                const int32_t* __restrict__ cu, int B, int64_t T,
                                                uint8_t* __restrict__ keep) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int b = find_prompt(cu, B, t);
  const SelState& s = st[b];
  uint8_t k = 1;
  if (t >= s.lo && t < s.hi) {
    const unsigned key = score_key(scores[t]);
    k = (key > s.theta || (key == s.theta && t <= (int64_t)s.idx_bound)) ? 1 : 0;
    if (s.theta == 0xffffffffu) k = 0;
  }
  keep[t] = k;
}

}  // namespace

size_t select_workspace_bytes(int B, int64_t /*T*/) {
  const size_t st = ((size_t)B * sizeof(SelState) + 255) & ~(size_t)255;
  return st + (size_t)B * kBins * sizeof(unsigned);
}

hipError_t launch_select(const float* scores, const int32_t* cu, const int32_t* db,
                         const int32_t* de, const int32_t* budget, int B, int64_t T,
                         uint8_t* keep, void* ws, hipStream_t s) {
  if (B == 0 || T == 0) return hipSuccess;
  auto* st = static_cast<SelState*>(ws);
  const size_t st_bytes = ((size_t)B * sizeof(SelState) + 255) & ~(size_t)255;
  auto* hist = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + st_bytes);
  hipLaunchKernelGGL(sel_init, dim3(B), dim3(256), 0, s, st, hist, cu, db, de, budget);
  const dim3 hgrid((unsigned)((T + kHistChunk - 1) / kHistChunk), (unsigned)B);
  for (int p = 0; p < 3; ++p) {
    hipLaunchKernelGGL(sel_hist, hgrid, dim3(kHistThreads), 0, s, scores, st, hist, p);
    hipLaunchKernelGGL(sel_pick, dim3(B), dim3(1024), 0, s, scores, st, hist, p);
  }
  hipLaunchKernelGGL(sel_mark, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, scores, st,
                     cu, B, T, keep);
  return hipGetLastError();
}

}  // namespace tg

// Document-only top-K selection (TokenGate article, section "How does
// TokenGate learned token pruning work?": a top-K selector keeps the
// highest-scoring tokens, only the document is prunable, the question never
// is).
//
// Order: score descending, then token index ascending.  Scores map to 32-bit
// keys whose unsigned order is that score order (-0.0 folded onto +0.0, every
// NaN onto key 0, below -inf).  Per prompt, an MSB-first radix select over
// three digits (11, 11, 10 bits) finds theta, the key of the k-th best
// document token, and how many tokens of key theta must be kept.  A token is
// kept when it lies outside the document, or its key is above theta, or its
// key equals theta and fewer than that many equal keys precede it.
//
// Up to 2^15 tokens, one workgroup per prompt runs the whole selection
// (sel_single): every pass re-reads the prompt's scores from L2, so there is
// one launch.  Longer inputs are cut into chunks of C tokens per prompt,
// from its first token, and take four kernels, all on the caller's stream,
// with no host sync, no atomics to global memory and no buffer that must
// start cleared:
//   sel_pass<0>  per (chunk, prompt): LDS histogram of digit 0 over the
//                chunk's document keys, written whole to the chunk's slot
//   sel_pass<1>, sel_pass<2>: every workgroup first sums the previous pass's
//                chunk histograms of its prompt and picks that digit (the same
//                result in every workgroup; the first one over the document
//                stores it for the next pass), then histograms the next digit
//                over the keys that match the digits picked so far
//   sel_mark     per (chunk, prompt): picks the last digit the same way, so
//                theta is exact; the last pass's chunk histograms also count
//                the keys equal to theta in each chunk, which ranks the equal
//                keys of a chunk among those of the whole document; writes
//                every keep flag of the chunk, question and template tokens
//                included
// Every count is an integer sum in a fixed order: the results do not depend
// on execution order.
#include <limits.h>

#include <atomic>

#include "tg_common.h"

// Scratch memory of the allocation-free entry point (tg_select_topk_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends,
// that takes the place of the caller's workspace (per-prompt states and chunk
// histograms).  The host never uses the array's name as a device address:
// its address on each device comes from hipGetSymbolAddress
// (tg::select_static_scratch).
static constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace tg {
namespace {

constexpr int kBins = 2048;
constexpr int kThreads = 1024;
constexpr int kMinChunk = 16384;  // tokens per workgroup
constexpr int kMaxChunks = 64;    // chunks per prompt at most (chunk size grows past that)
constexpr int kPer = kMinChunk / kThreads;  // keys per thread and round

// State of a prompt after the digits of passes < p are picked.
struct SelState {
  unsigned prefix;  // picked high bits of theta
  int k_rem;        // keys still to place at/below the prefix
  int pad[14];
};
static_assert(sizeof(SelState) == 64, "state size");

__device__ __forceinline__ unsigned score_key(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                     // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Digit p: bits [shift, shift + width).
__host__ __device__ constexpr int digit_shift(int p) { return p == 0 ? 21 : (p == 1 ? 10 : 0); }
__host__ __device__ constexpr unsigned digit_mask(int p) { return p == 2 ? 0x3ffu : 0x7ffu; }
// Bits fixed once the digits of passes < p are picked.
__host__ __device__ constexpr unsigned fixed_mask(int p) {
  return p == 0 ? 0u : (p == 1 ? 0xffe00000u : 0xfffffc00u);
}

// Per-workgroup view of its prompt and chunk.
struct Chunk {
  int pb, pe;    // prompt [pb, pe)
  int lo, hi;    // document [lo, hi)
  int k;         // document tokens to keep
  int mode;      // 0: keep no document token, 1: keep all, 2: radix select
  int c0, c1;    // this chunk [c0, c1)
  int x_first, x_last;  // chunks holding document tokens
  int slot0;     // slot of this prompt's chunk 0
};

// Sum over thread-held values of the workgroup (fixed order: wave sums,
// then the 16 wave totals in order).
__device__ int block_sum(int v, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) s += red[w];
  return s;
}

// Returns false when the chunk lies past the prompt (workgroup has nothing
// to do).  Uniform across the workgroup.
__device__ bool chunk_of(Chunk& c, const int32_t* cu, const int32_t* db, const int32_t* de,
                         const int32_t* budget, int C, int* red) {
  const int b = blockIdx.y;
  c.pb = cu[b];
  c.pe = cu[b + 1];
  const int64_t c0 = (int64_t)c.pb + (int64_t)blockIdx.x * C;
  if (c0 >= c.pe) return false;
  c.c0 = (int)c0;
  c.c1 = (int)min((int64_t)c.pe, c0 + C);
  c.lo = c.pb + db[b];
  c.hi = c.pb + de[b];
  const int n = c.hi - c.lo;
  c.k = min(budget[b], n);
  c.mode = c.k <= 0 ? 0 : (c.k >= n ? 1 : 2);
  c.x_first = (c.lo - c.pb) / C;
  c.x_last = n > 0 ? (c.hi - 1 - c.pb) / C : c.x_first - 1;
  // slots of earlier prompts: one per chunk of each
  int s = 0;
  for (int bb = threadIdx.x; bb < b; bb += kThreads) {
    const int len = cu[bb + 1] - cu[bb];
    s += (len + C - 1) / C;
  }
  c.slot0 = block_sum(s, red);
  return true;
}

// The digit of pass p from the chunk histograms of that pass: the bin where
// the count of keys in higher bins first reaches k_rem.  Thread j (counted
// from the top) owns bins 2047 - 2j and 2046 - 2j.  Returns the state after
// the pick; *n_bin is the count of the picked bin.
__device__ SelState pick_digit(int p, const SelState in, const unsigned* part, const Chunk& c,
                               unsigned* n_bin, unsigned* wtot, unsigned* s_res) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi_bin = kBins - 1 - 2 * tid;
  unsigned c_hi = 0u, c_lo = 0u;
  // both bins in one 8-byte load; eight chunks' loads in flight at once
  for (int x0 = c.x_first; x0 <= c.x_last; x0 += 8) {
    uint2 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = x0 + j <= c.x_last
                 ? *reinterpret_cast<const uint2*>(part + (size_t)(c.slot0 + x0 + j) * kBins + hi_bin - 1)
                 : make_uint2(0u, 0u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      c_lo += v[j].x;
      c_hi += v[j].y;
    }
  }
  const unsigned mine = c_hi + c_lo;
  unsigned incl = mine;  // inclusive scan over threads, top bins first
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  unsigned above = incl - mine;
  for (int w = 0; w < wave; ++w) above += wtot[w];
  const unsigned k_rem = (unsigned)in.k_rem;
  if (above < k_rem && k_rem <= above + mine) {
    // exactly one thread: the counts above its bins are < k_rem <= those
    // including them
    if (above + c_hi >= k_rem) {
      s_res[0] = (unsigned)hi_bin;
      s_res[1] = above;
      s_res[2] = c_hi;
    } else {
      s_res[0] = (unsigned)(hi_bin - 1);
      s_res[1] = above + c_hi;
      s_res[2] = c_lo;
    }
  }
  __syncthreads();
  SelState out = in;
  out.prefix = in.prefix | (s_res[0] << digit_shift(p));
  out.k_rem = in.k_rem - (int)s_res[1];
  *n_bin = s_res[2];
  return out;
}

// Pass P: pick digit P - 1 (P > 0), then histogram digit P over this chunk's
// document keys that match the digits picked so far.  Chunk histograms of
// pass P go to part[P & 1]; the state after pick P - 1 goes to st[P - 1].
template <int P>
__global__ __launch_bounds__(kThreads) void sel_pass(const float* __restrict__ scores,
                                                     const int32_t* cu, const int32_t* db,
                                                     const int32_t* de, const int32_t* budget,
                                                     int B, int C, SelState* st,
                                                     unsigned* part0, unsigned* part1) {
  __shared__ unsigned lh[kBins];
  __shared__ int red[kThreads / 64];
  __shared__ unsigned wtot[kThreads / 64];
  __shared__ unsigned s_res[3];
  Chunk c;
  if (!chunk_of(c, cu, db, de, budget, C, red)) return;
  if (c.mode != 2) return;
  const int b = blockIdx.y;
  const int x = blockIdx.x;
  const bool has_doc = x >= c.x_first && x <= c.x_last;  // uniform
  const int d0 = max(c.c0, c.lo), d1 = min(c.c1, c.hi);
  // The first round's scores do not depend on the digits picked so far:
  // their loads are issued before the pick, so the two memory round trips
  // overlap; the histogram is cleared before the pick's barriers too.
  float v[kPer];
  if (has_doc) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = d0 + (int)threadIdx.x + j * kThreads;
      v[j] = t < d1 ? scores[t] : 0.0f;
    }
    for (int i = threadIdx.x; i < kBins; i += kThreads) lh[i] = 0u;
  }
  SelState s;
  if (P == 0) {
    s.prefix = 0u;
    s.k_rem = c.k;
  } else {
    const SelState in = P == 1 ? SelState{0u, c.k, {0}} : st[(size_t)(P - 2) * B + b];
    unsigned n_bin;
    s = pick_digit(P - 1, in, (P - 1) & 1 ? part1 : part0, c, &n_bin, wtot, s_res);
    if (x == c.x_first && threadIdx.x == 0) st[(size_t)(P - 1) * B + b] = s;
  }
  if (!has_doc) return;  // no document token here
  __syncthreads();
  constexpr unsigned fm = fixed_mask(P);
  constexpr int sh = digit_shift(P);
  constexpr unsigned dm = digit_mask(P);
  // kPer keys per thread and round, all loads issued before the first use
  for (int r0 = d0; r0 < d1; r0 += kPer * kThreads) {
    if (r0 != d0) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int t = r0 + (int)threadIdx.x + j * kThreads;
        v[j] = t < d1 ? scores[t] : 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = r0 + (int)threadIdx.x + j * kThreads;
      const unsigned key = score_key(v[j]);
      if (t < d1 && (key & fm) == s.prefix) atomicAdd(&lh[(key >> sh) & dm], 1u);
    }
  }
  __syncthreads();
  unsigned* h = (P & 1 ? part1 : part0) + (size_t)(c.slot0 + x) * kBins;
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = lh[i];
}

// Keep flags of one chunk.  With the last digit picked, theta is exact and
// k_rem is the number of keys equal to theta that are kept, the first ones
// by index.  The equal keys before this chunk are counted from the last
// pass's chunk histograms (bin of theta's last digit); inside the chunk they
// are ranked in index order, 1024 tokens per step.
__global__ __launch_bounds__(kThreads) void sel_mark(const float* __restrict__ scores,
                                                     const int32_t* cu, const int32_t* db,
                                                     const int32_t* de, const int32_t* budget,
                                                     int B, int C, const SelState* st,
                                                     const unsigned* part0,
                                                     uint8_t* __restrict__ keep) {
  __shared__ int red[kThreads / 64];
  __shared__ unsigned wtot[kThreads / 64];
  __shared__ unsigned s_res[3];
  Chunk c;
  if (!chunk_of(c, cu, db, de, budget, C, red)) return;
  const int b = blockIdx.y;
  const int x = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned theta = 0u;
  int eq_keep = 0;   // equal keys kept (over the whole document)
  int eq_before = 0; // equal keys in the document's earlier chunks
  bool all_eq = true;
  // the first round's scores, loaded before the pick (they do not depend on
  // it), so the two memory round trips overlap
  float v[kPer];
  auto load_round = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = r0 + tid + j * kThreads;
      v[j] = (t < c.c1 && t >= c.lo && t < c.hi) ? scores[t] : 0.0f;
    }
  };
  if (c.mode == 2) load_round(c.c0);
  if (c.mode == 2) {
    unsigned n_eq;
    const SelState s = pick_digit(2, st[(size_t)B + b], part0, c, &n_eq, wtot, s_res);
    theta = s.prefix;
    eq_keep = s.k_rem;
    all_eq = (unsigned)eq_keep >= n_eq;
    if (!all_eq) {
      const unsigned bin = theta & digit_mask(2);
      int e = 0;  // at most kMaxChunks terms: one load per thread
      for (int xx = c.x_first + tid; xx < x; xx += kThreads)
        e += (int)part0[(size_t)(c.slot0 + xx) * kBins + bin];
      eq_before = block_sum(e, red);
    }
  }
  // kPer tokens per thread and round (token r0 + tid + j * kThreads), the
  // score loads all issued before the first use; index order within a round
  // is (j, tid)
  for (int r0 = c.c0; r0 < c.c1; r0 += kPer * kThreads) {
    if (c.mode == 2 && r0 != c.c0) load_round(r0);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int t = r0 + tid + j * kThreads;
      const bool in = t < c.c1;
      const bool doc = in && t >= c.lo && t < c.hi;
      uint8_t k = 1;
      bool eq = false;
      if (doc) {
        if (c.mode == 0) {
          k = 0;
        } else if (c.mode == 2) {
          const unsigned key = score_key(v[j]);
          k = key > theta ? 1 : 0;
          eq = key == theta;
          if (eq && all_eq) k = 1;
        }
      }
      if (!all_eq) {  // uniform: rank the equal keys of this step
        const unsigned long long bal = __ballot(eq);
        const int in_wave = __popcll(bal & ((lane == 63) ? ~0ull : ((2ull << lane) - 1)));
        __syncthreads();
        if (lane == 63) wtot[wave] = (unsigned)in_wave;
        __syncthreads();
        int before = 0, round_total = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
          if (w < wave) before += (int)wtot[w];
          round_total += (int)wtot[w];
        }
        if (eq) k = (eq_before + before + in_wave <= eq_keep) ? 1 : 0;
        eq_before += round_total;
      }
      if (in) keep[t] = k;
    }
  }
}

// Whole selection of one prompt in one workgroup (inputs up to
// kSingleMaxT tokens): the same three digits and the same keep rule, with
// the histograms in LDS and the scores re-read from L2 on every pass, so
// there is one launch and no workspace.  Each digit value has four
// sub-bins (chosen by lane % 4), which spreads the atomics of equal digits
// in one wave over four addresses; the pick adds them back.
constexpr int kSub = 4;
constexpr int64_t kSingleMaxT = (int64_t)1 << 15;
constexpr int kSPer = 16;  // keys per thread and round, all loads in flight

__global__ __launch_bounds__(kThreads) void sel_single(const float* __restrict__ scores,
                                                       const int32_t* cu, const int32_t* db,
                                                       const int32_t* de, const int32_t* budget,
                                                       uint8_t* __restrict__ keep) {
  __shared__ unsigned lh[kBins * kSub];
  __shared__ unsigned wtot[kThreads / 64];
  __shared__ unsigned s_res[3];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pb = cu[b], pe = cu[b + 1];
  const int lo = pb + db[b], hi = pb + de[b];
  const int n = hi - lo;
  const int k = min(budget[b], n);
  const int mode = k <= 0 ? 0 : (k >= n ? 1 : 2);

  unsigned theta = 0u;
  int eq_keep = 0;
  bool all_eq = true;
  if (mode == 2) {
    unsigned prefix = 0u;
    int k_rem = k;
    unsigned n_bin = 0u;
    for (int p = 0; p < 3; ++p) {
      const unsigned fm = fixed_mask(p);
      const int sh = digit_shift(p);
      const unsigned dm = digit_mask(p);
      for (int i = tid; i < kBins * kSub; i += kThreads) lh[i] = 0u;
      __syncthreads();
      for (int r0 = lo; r0 < hi; r0 += kSPer * kThreads) {
        float v[kSPer];
#pragma unroll
        for (int j = 0; j < kSPer; ++j) {
          const int t = r0 + tid + j * kThreads;
          v[j] = t < hi ? scores[t] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kSPer; ++j) {
          const int t = r0 + tid + j * kThreads;
          const unsigned key = score_key(v[j]);
          if (t < hi && (key & fm) == prefix)
            atomicAdd(&lh[((key >> sh) & dm) * kSub + (lane & (kSub - 1))], 1u);
        }
      }
      __syncthreads();
      // pick: thread j (counted from the top) owns bins 2047 - 2j and 2046 - 2j
      const int hi_bin = kBins - 1 - 2 * tid;
      unsigned c_hi = 0u, c_lo = 0u;
#pragma unroll
      for (int q = 0; q < kSub; ++q) {
        c_hi += lh[hi_bin * kSub + q];
        c_lo += lh[(hi_bin - 1) * kSub + q];
      }
      const unsigned mine = c_hi + c_lo;
      unsigned incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane == 63) wtot[wave] = incl;
      __syncthreads();
      unsigned above = incl - mine;
      for (int w = 0; w < wave; ++w) above += wtot[w];
      const unsigned kr = (unsigned)k_rem;
      if (above < kr && kr <= above + mine) {  // exactly one thread
        if (above + c_hi >= kr) {
          s_res[0] = (unsigned)hi_bin;
          s_res[1] = above;
          s_res[2] = c_hi;
        } else {
          s_res[0] = (unsigned)(hi_bin - 1);
          s_res[1] = above + c_hi;
          s_res[2] = c_lo;
        }
      }
      __syncthreads();
      prefix |= s_res[0] << sh;
      k_rem -= (int)s_res[1];
      n_bin = s_res[2];
      __syncthreads();  // s_res and wtot are written again in the next pass
    }
    theta = prefix;
    eq_keep = k_rem;
    all_eq = (unsigned)eq_keep >= n_bin;
  }

  // keep flags of the whole prompt; equal keys ranked in index order
  int eq_before = 0;
  for (int r0 = pb; r0 < pe; r0 += kSPer * kThreads) {
    float v[kSPer];
    if (mode == 2) {
#pragma unroll
      for (int j = 0; j < kSPer; ++j) {
        const int t = r0 + tid + j * kThreads;
        v[j] = (t < pe && t >= lo && t < hi) ? scores[t] : 0.0f;
      }
    }
#pragma unroll
    for (int j = 0; j < kSPer; ++j) {
      const int t = r0 + tid + j * kThreads;
      const bool in = t < pe;
      const bool doc = in && t >= lo && t < hi;
      uint8_t kf = 1;
      bool eq = false;
      if (doc) {
        if (mode == 0) {
          kf = 0;
        } else if (mode == 2) {
          const unsigned key = score_key(v[j]);
          kf = key > theta ? 1 : 0;
          eq = key == theta;
          if (eq && all_eq) kf = 1;
        }
      }
      if (!all_eq) {  // uniform: rank the equal keys of this step
        const unsigned long long bal = __ballot(eq);
        const int in_wave = __popcll(bal & ((lane == 63) ? ~0ull : ((2ull << lane) - 1)));
        __syncthreads();
        if (lane == 63) wtot[wave] = (unsigned)in_wave;
        __syncthreads();
        int before = 0, step_total = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
          if (w < wave) before += (int)wtot[w];
          step_total += (int)wtot[w];
        }
        if (eq) kf = (eq_before + before + in_wave <= eq_keep) ? 1 : 0;
        eq_before += step_total;
      }
      if (in) keep[t] = kf;
    }
  }
}

int chunk_size(int64_t T) {
  int64_t C = kMinChunk;
  while ((T + C - 1) / C > kMaxChunks) C *= 2;
  return (int)C;
}

size_t n_slots(int B, int64_t T) { return (size_t)((T + chunk_size(T) - 1) / chunk_size(T)) + (size_t)B; }

}  // namespace

size_t select_static_scratch_capacity() { return kStaticScratchBytes; }

size_t select_scratch_bytes_needed(int B, int64_t T) {
  // the one-workgroup path uses no workspace
  return (B == 0 || T == 0 || T <= kSingleMaxT) ? 0 : select_workspace_bytes(B, T);
}

hipError_t select_static_scratch(hipStream_t stream, void** ptr) {
  // The array of the device the stream belongs to (the current device for
  // the null stream), resolved once per device with that device current;
  // concurrent first calls resolve and store the same address.
  static std::atomic<void*> addr[64];
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

size_t select_workspace_bytes(int B, int64_t T) {
  const size_t st = ((size_t)2 * B * sizeof(SelState) + 255) & ~(size_t)255;
  return st + 2 * n_slots(B, T) * kBins * sizeof(unsigned);
}

hipError_t launch_select(const float* scores, const int32_t* cu, const int32_t* db,
                         const int32_t* de, const int32_t* budget, int B, int64_t T,
                         uint8_t* keep, void* ws, hipStream_t s) {
  if (B == 0 || T == 0) return hipSuccess;
  if (T <= kSingleMaxT) {
    hipLaunchKernelGGL(sel_single, dim3((unsigned)B), dim3(kThreads), 0, s, scores, cu, db, de,
                       budget, keep);
    return hipGetLastError();
  }
  auto* st = static_cast<SelState*>(ws);
  const size_t st_bytes = ((size_t)2 * B * sizeof(SelState) + 255) & ~(size_t)255;
  auto* part0 = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + st_bytes);
  auto* part1 = part0 + n_slots(B, T) * kBins;
  const int C = chunk_size(T);
  const dim3 grid((unsigned)((T + C - 1) / C), (unsigned)B);
  hipLaunchKernelGGL(sel_pass<0>, grid, dim3(kThreads), 0, s, scores, cu, db, de, budget, B, C, st,
                     part0, part1);
  hipLaunchKernelGGL(sel_pass<1>, grid, dim3(kThreads), 0, s, scores, cu, db, de, budget, B, C, st,
                     part0, part1);
  hipLaunchKernelGGL(sel_pass<2>, grid, dim3(kThreads), 0, s, scores, cu, db, de, budget, B, C, st,
                     part0, part1);
  hipLaunchKernelGGL(sel_mark, grid, dim3(kThreads), 0, s, scores, cu, db, de, budget, B, C, st,
                     part0, keep);
  return hipGetLastError();
}

}  // namespace tg

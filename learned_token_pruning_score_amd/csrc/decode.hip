// Decode over the kept-only KV cache (TokenGate article, section "How does
// TokenGate learned token pruning work?": the layers above the gate never
// create KV entries for pruned tokens, so generation reads only the kept
// ones; "What is token-gated attention?": a kept token's score is its
// attention bias).  The bias is persistent: document keys keep their gate
// score, question and generated keys carry 0.
//
// Cache layout (per pruned layer): rows [rows, Hkv, d] for k and v with
// token strides, a bias per row (fp32); sequence b owns rows start[b] ..
// start[b] + len[b] - 1, with room after them for the tokens it generates.
//   kv_scatter   prefill's compacted rows (ragged by cu_kept) into the cache,
//                in 16-byte units when alignment and strides allow.
//   kv_append    each step's new k, v at row start[b] + pos[b], bias 0.
//   decode_split one workgroup of 4 waves per (sequence, KV head, split of 128
//                keys, 256 once the grid holds about 8 workgroups per CU): a
//                decode step reads every cached key once and does
//                Hq/Hkv dot products per key, so it is bound by HBM, not by the
//                matrix cores: 16 lanes (d = 128; 8 for d = 64) share one key
//                row (16 bytes each, one coalesced read), the group's queries
//                sit in registers, and every lane group runs an online softmax
//                over its keys; the groups of a wave and the waves of the
//                workgroup merge in a fixed order into one (max, sum, o)
//                partial per query head.
//   decode_merge the splits' partials merged per (sequence, head): one wave
//                per 4 output elements, lanes over the splits, fixed-order
//                butterflies: bit-reproducible, no atomics.
#include <math.h>

#include <algorithm>

#include "tg_common.h"

namespace tg {
namespace {

constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;
constexpr int kSplit = 128;      // keys per split
constexpr int kSplitLong = 256;  // keys per split once the grid holds about 8 workgroups per CU

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename T>
__device__ __forceinline__ T from_float(float x) {
  if constexpr (sizeof(T) == 2) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return x;
}

// (m1, l1, o1) <- merge with (m2, l2, o2); m in log2 units, -inf = empty.
__device__ __forceinline__ void merge_state(float& m1, float& l1, float* o1, float m2, float l2, const float* o2, int n) {
  const float M = fmaxf(m1, m2);
  const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - M);
  const float a2 = m2 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m2 - M);
  l1 = l1 * a1 + l2 * a2;
  for (int e = 0; e < n; ++e) o1[e] = o1[e] * a1 + o2[e] * a2;
  m1 = M;
}

template <typename T>
__global__ __launch_bounds__(256) void kv_scatter_kernel(const T* __restrict__ k, const T* __restrict__ v, int64_t sks,
                                                         int64_t svs, const float* __restrict__ bias,
                                                         const int32_t* __restrict__ cu, int B, int64_t Kt, int Hkv,
                                                         int d, T* __restrict__ kc, T* __restrict__ vc, int64_t ks,
                                                         int64_t vs, float* __restrict__ bc,
                                                         const int32_t* __restrict__ start) {
  const int64_t row_elems = (int64_t)Hkv * d;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Kt * row_elems) return;
  const int64_t r = i / row_elems;
  const int64_t e = i - r * row_elems;
  int lo = 0, hi = B;  // prompt b with cu[b] <= r < cu[b + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (cu[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int64_t dst = (int64_t)start[lo] + (r - cu[lo]);
  kc[dst * ks + e] = k[r * sks + e];
  vc[dst * vs + e] = v[r * svs + e];
  if (e == 0) bc[dst] = bias ? bias[r] : 0.0f;
}

// The same copy in 16-byte units (pointers 16-byte aligned, strides and the
// row's Hkv * d elements a whole number of 16-byte units): thread i moves
// unit i % row_units of kept row i / row_units, all in bytes.
__global__ __launch_bounds__(256) void kv_scatter16_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                           int64_t sks, int64_t svs, const float* __restrict__ bias,
                                                           const int32_t* __restrict__ cu, int B, int64_t Kt,
                                                           int row_units, char* __restrict__ kc, char* __restrict__ vc,
                                                           int64_t ks, int64_t vs, float* __restrict__ bc,
                                                           const int32_t* __restrict__ start) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Kt * row_units) return;
  const int64_t r = i / row_units;
  const int64_t e = (i - r * row_units) * 16;
  int lo = 0, hi = B;  // prompt b with cu[b] <= r < cu[b + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (cu[mid] <= r) lo = mid;
    else hi = mid;
  }
  const int64_t dst = (int64_t)start[lo] + (r - cu[lo]);
  *reinterpret_cast<uint4*>(kc + dst * ks + e) = *reinterpret_cast<const uint4*>(k + r * sks + e);
  *reinterpret_cast<uint4*>(vc + dst * vs + e) = *reinterpret_cast<const uint4*>(v + r * svs + e);
  if (e == 0) bc[dst] = bias ? bias[r] : 0.0f;
}

template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(const T* __restrict__ kn, const T* __restrict__ vn, int B,
                                                        int Hkv, int d, T* __restrict__ kc, T* __restrict__ vc,
                                                        int64_t ks, int64_t vs, float* __restrict__ bc,
                                                        const int32_t* __restrict__ start, const int32_t* __restrict__ pos) {
  const int64_t row_elems = (int64_t)Hkv * d;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)B * row_elems) return;
  const int b = (int)(i / row_elems);
  const int64_t e = i - (int64_t)b * row_elems;
  const int64_t dst = (int64_t)start[b] + pos[b];
  kc[dst * ks + e] = kn[i];
  vc[dst * vs + e] = vn[i];
  if (e == 0) bc[dst] = 0.0f;  // generated keys carry no bias
}

// Partial of one split.  part_m / part_l [B * Hq, n_split], part_o [B * Hq,
// n_split, HD]; grid (B * Hkv, n_split).
template <typename T, int HD, int G, int KS>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc, int64_t ks, int64_t vs,
    const float* __restrict__ bc, const float* __restrict__ gain, float c2, const int32_t* __restrict__ start,
    const int32_t* __restrict__ lens, int Hq, int Hkv, int n_split, float* __restrict__ part_m,
    float* __restrict__ part_l, float* __restrict__ part_o) {
  constexpr int LPK = HD / 8;       // lanes per key
  constexpr int KPW = 64 / LPK;     // keys per wave step
  constexpr int KW = KS / 4;        // keys per wave per split
  __shared__ float sm[4][G], sl[4][G], so[4][G][HD];
  const int b = blockIdx.x / Hkv;
  const int kvh = blockIdx.x - b * Hkv;
  const int split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane / LPK;        // key group of the lane
  const int sub = lane % LPK;       // its 8 elements: [8 sub, 8 sub + 8)
  const int n = lens[b];
  const int64_t base = start[b];
  if ((int64_t)split * KS >= n) {
    // no key of the sequence in this split (ragged caches): the empty
    // partial (max -inf, sum 0, o 0), without the loads and the loop
    for (int idx = tid; idx < G * HD; idx += 256) {
      const int g = idx / HD, e = idx - g * HD;
      const int64_t ph = ((int64_t)b * Hq + kvh * G + g) * n_split + split;
      part_o[ph * HD + e] = 0.0f;
      if (e == 0) {
        part_m[ph] = -INFINITY;
        part_l[ph] = 0.0f;
      }
    }
    return;
  }
  // queries of the group, pre-scaled to log2 units
  float qv[G][8], gb[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int h = kvh * G + g;
    load8(q + ((int64_t)b * Hq + h) * HD + 8 * sub, qv[g]);
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[g][j] *= c2;
    gb[g] = (gain && bc) ? gain[h] * kLog2eD : 0.0f;
  }
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = 0.0f;
  }
  // keys in batches of NB per lane group: the loads of a batch are all
  // issued before any of its keys is used; a batch never reaches past the
  // wave's KW keys
  constexpr int NB0 = sizeof(T) == 2 ? 4 : 2;
  constexpr int NB = KW / KPW < NB0 ? KW / KPW : NB0;
  static_assert(NB >= 1 && KW % (KPW * NB) == 0, "a wave's keys split into whole batches");
  const int k_lo = split * KS + wave * KW;
  for (int kk = 0; kk < KW; kk += KPW * NB) {
    float kv8[NB][8], vv8[NB][8], sb[NB];
    bool ok[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int key = k_lo + kk + u * KPW + kg;
      ok[u] = key < n;  // uniform within the lane's key group
      const int64_t row = base + (ok[u] ? key : 0);
      load8(kc + row * ks + (int64_t)kvh * HD + 8 * sub, kv8[u]);
      load8(vc + row * vs + (int64_t)kvh * HD + 8 * sub, vv8[u]);
      sb[u] = bc ? bc[row] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (ok[u]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float dot = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) dot = fmaf(qv[g][j], kv8[u][j], dot);
#pragma unroll
          for (int off = 1; off < LPK; off <<= 1) dot += __shfl_xor(dot, off);
          const float x = fmaf(gb[g], sb[u], dot);
          const float mn = fmaxf(m[g], x);
          const float a = __builtin_amdgcn_exp2f(m[g] - mn);  // m = -inf: 0
          const float p = __builtin_amdgcn_exp2f(x - mn);
          l[g] = l[g] * a + p;
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] = fmaf(o[g][j], a, p * vv8[u][j]);
          m[g] = mn;
        }
      }
    }
  }
  // merge the key groups of the wave (lanes sub, sub + LPK, ...), fixed butterfly
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(m[g], off), l2 = __shfl_xor(l[g], off);
      float o2[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o2[j] = __shfl_xor(o[g][j], off);
      merge_state(m[g], l[g], o[g], m2, l2, o2, 8);
    }
  }
  if (kg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (sub == 0) {
        sm[wave][g] = m[g];
        sl[wave][g] = l[g];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) so[wave][g][8 * sub + j] = o[g][j];
    }
  }
  __syncthreads();
  // waves 0..3 in order; thread (g, e) merges element e of head g
  for (int idx = tid; idx < G * HD; idx += 256) {
    const int g = idx / HD, e = idx - g * HD;
    float M = sm[0][g], L = sl[0][g], O = so[0][g][e];
    for (int w = 1; w < 4; ++w) merge_state(M, L, &O, sm[w][g], sl[w][g], &so[w][g][e], 1);
    const int64_t ph = ((int64_t)b * Hq + kvh * G + g) * n_split + split;
    part_o[ph * HD + e] = O;
    if (e == 0) {
      part_m[ph] = M;
      part_l[ph] = L;
    }
  }
}

// The splits' partials of one (sequence, head) merged in two passes, every
// load independent of the arithmetic before it: the overall max M, then
// sum_s l_s 2^(m_s - M) and sum_s o_s 2^(m_s - M).
template <typename T, int HD>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_m, const float* __restrict__ part_l,
                                                           const float* __restrict__ part_o, int64_t BH, int n_split,
                                                           T* __restrict__ out, float* __restrict__ lse) {
  // one wave per (sequence-head bh, 4 consecutive output elements); lane l
  // takes the splits l, l + 64, ..., so every partial is loaded in one batch,
  // and the max and the sums over the lanes are fixed-order butterflies
  constexpr int NC = HD / 4;
  const int64_t wid = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;  // wave-uniform
  const int lane = threadIdx.x & 63;
  if (wid >= BH * NC) return;
  const int64_t bh = wid / NC;
  const int c = (int)(wid - bh * NC);
  const float* pm = part_m + bh * n_split;
  const float* pl = part_l + bh * n_split;
  const float* po = part_o + bh * n_split * HD + 4 * c;
  float M = -INFINITY;
  for (int s = lane; s < n_split; s += 64) M = fmaxf(M, pm[s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.0f, O[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s = lane; s < n_split; s += 64) {
    const float w = __builtin_amdgcn_exp2f(pm[s] - M);  // empty split: 2^-inf = 0
    const float4 o = *reinterpret_cast<const float4*>(po + (int64_t)s * HD);
    L = fmaf(pl[s], w, L);
    O[0] = fmaf(o.x, w, O[0]);
    O[1] = fmaf(o.y, w, O[1]);
    O[2] = fmaf(o.z, w, O[2]);
    O[3] = fmaf(o.w, w, O[3]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    L += __shfl_xor(L, off);
#pragma unroll
    for (int j = 0; j < 4; ++j) O[j] += __shfl_xor(O[j], off);
  }
  if (lane < 4) out[bh * HD + 4 * c + lane] = from_float<T>(O[lane] / L);  // an empty sequence gives NaN
  if (lane == 0 && c == 0 && lse) lse[bh] = (M + __log2f(L)) * kLn2D;
}

size_t dalign(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T, int HD>
hipError_t launch_split(int G, bool long_split, dim3 grid, hipStream_t s, const T* q, const T* kc, const T* vc,
                        int64_t ks, int64_t vs, const float* bc, const float* gain, float c2, const int32_t* start,
                        const int32_t* lens, int Hq, int Hkv, int n_split, float* pm, float* pl, float* po) {
#define TG_DEC(GG)                                                                                                   \
  if (long_split)                                                                                                    \
    hipLaunchKernelGGL((decode_split_kernel<T, HD, GG, kSplitLong>), grid, dim3(256), 0, s, q, kc, vc, ks, vs, bc,  \
                       gain, c2, start, lens, Hq, Hkv, n_split, pm, pl, po);                                         \
  else                                                                                                               \
    hipLaunchKernelGGL((decode_split_kernel<T, HD, GG, kSplit>), grid, dim3(256), 0, s, q, kc, vc, ks, vs, bc, gain, \
                       c2, start, lens, Hq, Hkv, n_split, pm, pl, po)
  switch (G) {
    case 1: TG_DEC(1); break;
    case 2: TG_DEC(2); break;
    case 3: TG_DEC(3); break;
    case 4: TG_DEC(4); break;
    case 5: TG_DEC(5); break;
    case 6: TG_DEC(6); break;
    case 7: TG_DEC(7); break;
    case 8: TG_DEC(8); break;
    default: return hipErrorInvalidValue;
  }
#undef TG_DEC
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int B, int Hq, int d, int max_len) {
  const int64_t n_split = std::max(1, (max_len + kSplit - 1) / kSplit);
  const int64_t P = (int64_t)B * Hq * n_split;
  return 2 * dalign((size_t)P * 4) + dalign((size_t)P * d * 4);
}

hipError_t launch_kv_scatter(const void* k, const void* v, int64_t sks, int64_t svs, const float* bias,
                             const int32_t* cu, int B, int64_t Kt, int Hkv, int d, int elem_bytes, void* kc,
                             void* vc, int64_t ks, int64_t vs, float* bc, const int32_t* start, hipStream_t s) {
  const int64_t total = Kt * Hkv * d;
  if (total == 0) return hipSuccess;
  const int64_t row_bytes = (int64_t)Hkv * d * elem_bytes;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (row_bytes % 16 == 0 && (sks * elem_bytes) % 16 == 0 && (svs * elem_bytes) % 16 == 0 &&
      (ks * elem_bytes) % 16 == 0 && (vs * elem_bytes) % 16 == 0 && a16(k) && a16(v) && a16(kc) && a16(vc)) {
    const int row_units = (int)(row_bytes / 16);
    const int64_t n = Kt * row_units;
    hipLaunchKernelGGL(kv_scatter16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const char*>(k), static_cast<const char*>(v), sks * elem_bytes, svs * elem_bytes,
                       bias, cu, B, Kt, row_units, static_cast<char*>(kc), static_cast<char*>(vc), ks * elem_bytes,
                       vs * elem_bytes, bc, start);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((total + 255) / 256));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(kv_scatter_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), sks, svs, bias, cu, B, Kt, Hkv, d, static_cast<uint16_t*>(kc),
                       static_cast<uint16_t*>(vc), ks, vs, bc, start);
  else
    hipLaunchKernelGGL(kv_scatter_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(k),
                       static_cast<const float*>(v), sks, svs, bias, cu, B, Kt, Hkv, d, static_cast<float*>(kc),
                       static_cast<float*>(vc), ks, vs, bc, start);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* kn, const void* vn, int B, int Hkv, int d, int elem_bytes, void* kc, void* vc,
                            int64_t ks, int64_t vs, float* bc, const int32_t* start, const int32_t* pos, hipStream_t s) {
  const int64_t total = (int64_t)B * Hkv * d;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (elem_bytes == 2)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(kn),
                       static_cast<const uint16_t*>(vn), B, Hkv, d, static_cast<uint16_t*>(kc),
                       static_cast<uint16_t*>(vc), ks, vs, bc, start, pos);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(kn),
                       static_cast<const float*>(vn), B, Hkv, d, static_cast<float*>(kc), static_cast<float*>(vc), ks,
                       vs, bc, start, pos);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const void* q, const void* kc, const void* vc, int64_t ks, int64_t vs, const float* bc,
                              const float* gain, float tau, const int32_t* start, const int32_t* lens, int B,
                              int max_len, int Hq, int Hkv, int d, int elem_bytes, void* out, float* lse, void* ws,
                              hipStream_t s) {
  // longer splits once there are enough workgroups (fewer partials to write
  // and merge); the workspace is sized for the shorter ones, the larger count
  const bool long_split = (int64_t)B * Hkv * ((max_len + kSplitLong - 1) / kSplitLong) >= 2048;
  const int split_keys = long_split ? kSplitLong : kSplit;
  const int n_split = std::max(1, (max_len + split_keys - 1) / split_keys);
  const int64_t P = (int64_t)B * Hq * n_split;
  char* w = static_cast<char*>(ws);
  float* pm = reinterpret_cast<float*>(w);
  float* pl = reinterpret_cast<float*>(w + dalign((size_t)P * 4));
  float* po = reinterpret_cast<float*>(w + 2 * dalign((size_t)P * 4));
  const int G = Hq / Hkv;
  const float c2 = tau / sqrtf((float)d) * kLog2eD;
  const dim3 grid((unsigned)(B * Hkv), (unsigned)n_split);
  hipError_t e;
  if (elem_bytes == 2) {
    const auto* qp = static_cast<const uint16_t*>(q);
    const auto* kp = static_cast<const uint16_t*>(kc);
    const auto* vp = static_cast<const uint16_t*>(vc);
    e = d == 128 ? launch_split<uint16_t, 128>(G, long_split, grid, s, qp, kp, vp, ks, vs, bc, gain, c2, start, lens, Hq, Hkv, n_split, pm, pl, po)
                 : launch_split<uint16_t, 64>(G, long_split, grid, s, qp, kp, vp, ks, vs, bc, gain, c2, start, lens, Hq, Hkv, n_split, pm, pl, po);
  } else {
    const auto* qp = static_cast<const float*>(q);
    const auto* kp = static_cast<const float*>(kc);
    const auto* vp = static_cast<const float*>(vc);
    e = d == 128 ? launch_split<float, 128>(G, long_split, grid, s, qp, kp, vp, ks, vs, bc, gain, c2, start, lens, Hq, Hkv, n_split, pm, pl, po)
                 : launch_split<float, 64>(G, long_split, grid, s, qp, kp, vp, ks, vs, bc, gain, c2, start, lens, Hq, Hkv, n_split, pm, pl, po);
  }
  if (e != hipSuccess) return e;
  const int64_t BH = (int64_t)B * Hq;
  const dim3 mg((unsigned)((BH * (d / 4) * 64 + 255) / 256));  // one wave per 4 output elements
  if (elem_bytes == 2) {
    if (d == 128) hipLaunchKernelGGL((decode_merge_kernel<uint16_t, 128>), mg, dim3(256), 0, s, pm, pl, po, BH, n_split, static_cast<uint16_t*>(out), lse);
    else hipLaunchKernelGGL((decode_merge_kernel<uint16_t, 64>), mg, dim3(256), 0, s, pm, pl, po, BH, n_split, static_cast<uint16_t*>(out), lse);
  } else {
    if (d == 128) hipLaunchKernelGGL((decode_merge_kernel<float, 128>), mg, dim3(256), 0, s, pm, pl, po, BH, n_split, static_cast<float*>(out), lse);
    else hipLaunchKernelGGL((decode_merge_kernel<float, 64>), mg, dim3(256), 0, s, pm, pl, po, BH, n_split, static_cast<float*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace tg

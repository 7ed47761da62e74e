// Backward of token-gated attention (TokenGate article, section "What is
// token-gated attention?": top-K selection is not differentiable, so each
// kept token's score enters the attention above the gate as a logit bias,
// which gives the loss a gradient path back to the scorer; the per-head gain
// and the temperature are learned too).  With
//     x_ij = tau q_i.k_j / sqrt(d) + g_h s_j   (keys j <= i of i's prompt)
//     P = softmax_j(x),  o_i = sum_j P_ij v_j,  D_i = dout_i . o_i
//     dx_ij = P_ij (dout_i . v_j - D_i)
// the gradients are
//     dq_i = tau/sqrt(d) sum_j dx_ij k_j          (per query head)
//     dk_j = tau/sqrt(d) sum_(h in group, i) dx_ij q_i
//     dv_j = sum_(h in group, i) P_ij dout_i
//     ds_j = sum_h g_h c_hj,  dg_h = sum_j s_j c_hj,  with c_hj = sum_i dx_ij
//     dtau = sum_(h, ij) dx_ij q_i.k_j / sqrt(d)
// P is recomputed from the forward's log-sum-exp.  Every sum runs in a fixed
// order (no atomics), so the results are bit-reproducible:
//   bwd_prep   D_i per (row, head).
//   bwd_dq     query-parallel, the forward's layout: one workgroup of 4 waves
//              per (head, prompt, 128-row query tile), 32 rows per wave; for
//              each 64-key tile S^T = K Q^T and dP^T = V dO^T on the 32x32x16
//              bf16 MFMA (lane = query, keys in registers), dx^T in fp32,
//              dQ^T += K^T dx^T with a transposing LDS read of K (the
//              forward's value product); partial sums of dx q.k for dtau.
//   bwd_dkdv   key-parallel: one workgroup of 4 waves per (KV head, prompt,
//              128-key tile), 32 keys per wave; for each head of the group and
//              each 64-row query tile S = Q K^T (lane = key, queries in
//              registers), then in one pass dV^T += dO^T P, in a second
//              dP = dO V^T and dK^T += Q^T dx with transposing reads of dO and
//              Q; column sums c_hj of dx in fp32.
//   bwd_final  ds and dg from c_hj, dtau from the partial sums.
// fp32 path: one thread per (query, head) for dq and per (key, KV head) for
// dk / dv, on vector ALUs.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "tg_common.h"

namespace tg {
namespace {

constexpr float kLog2eB = 1.4426950408889634f;
constexpr int kBufFlagsB = 0x00020000;  // raw buffer: reads past num_records give 0
constexpr int kT = 64;                  // rows per staged tile (keys in bwd_dq, queries in bwd_dkdv)

typedef short s4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4v lds_s4v;
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const u32x4v lds_u4v;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(reinterpret_cast<const char*>(p));
}

// 16-byte fragment of a row-major staged tile, read from a per-lane base
// address (row lane % 32, 16-byte unit lane / 32) plus a compile-time byte
// offset (rows and units further on), which the LDS instruction carries as
// its immediate: one address register per staged tile instead of one per
// read.
__device__ __forceinline__ bf16x8 frag_at(uint32_t lane_base, uint32_t off) {
  return __builtin_bit_cast(bf16x8, *(lds_u4v*)(uintptr_t)(lane_base + off));
}

// A pointer every lane of the wave holds, moved to scalar registers so that
// the buffer descriptors built from it are known to be uniform.
template <typename T>
__device__ __forceinline__ const T* wave_uniform(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Transposed fragment of a row-major staged tile with rows of ROWT 16-byte
// units (the forward's value-product read): within each 16-lane group,
// lane i receives element i % 4 of the 8-byte chunks addressed by lanes
// 4j + i / 4.  Lane s of group g addresses row 4 (g / 2) + s / 4 and columns
// 16 (g % 2) + 4 (s % 4) .. +3 of a 16-row step, so lane l receives rows
// 4G..4G+3 (then +8..+11) of column l % 32 of the 32-column block: the
// A operand of an MFMA whose k index runs over the staged rows in the order
// the score accumulator holds them.  kh: 16-row step (0..3), db: 32-column
// block.
template <int ROWT>
__device__ __forceinline__ bf16x8 frag_tr(uint32_t tbase, int kh, int db) {
  const uint32_t a0 = tbase + ((kh >> 1) * 32 + 16 * (kh & 1)) * (ROWT * 16) + db * 64;
  const s4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(uintptr_t)a0);
  const s4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4v*)(uintptr_t)(a0 + 8 * (ROWT * 16)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int ROWT>
__device__ __forceinline__ uint32_t tr_lane_base(const void* tile, int lane) {
  const int gi = lane & 15, g = lane >> 4;
  return lds_addr(reinterpret_cast<const char*>(tile) + (4 * (g >> 1) + (gi >> 2)) * (ROWT * 16) +
                  (16 * (g & 1) + 4 * (gi & 3)) * 2);
}

// accumulator (two 32-row blocks) -> B operand of the second product, rows
// relabelled as in frag_tr: pb[kb][hh] holds registers 8 hh .. 8 hh + 7
__device__ __forceinline__ void to_b_operand(const float (&v)[2][16], bf16x8 (&pb)[2][2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[kb][hh][j] = (__bf16)v[kb][8 * hh + j];
}

// One row's 32 columns of an accumulator block, scaled by mul, as bf16 at p
// (16-byte stores, store_row32_bf16); only `store` lanes write.
__device__ __forceinline__ void store_bf16_rows(uint16_t* p, const f32x16& a, float mul, int G, bool store) {
  store_row32_bf16(p, G, store, [&](int i) __attribute__((always_inline)) { return a[i] * mul; });
}

// Fixed-order wave sum (butterfly over the 64 lanes).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// D[h][i] = dout_i . o_i for fp32 inputs, one thread per (row, head).
__global__ __launch_bounds__(256) void bwd_prep_f32_kernel(const float* __restrict__ o, const float* __restrict__ dout,
                                                           int64_t Kt, int Hq, int d, float* __restrict__ D) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= Kt * Hq) return;
  const int64_t i = idx / Hq;
  const int h = (int)(idx - i * Hq);
  const float* op = o + idx * d;
  const float* gp = dout + idx * d;
  float acc = 0.0f;
  for (int e = 0; e < d; ++e) acc = fmaf(op[e], gp[e], acc);
  D[(int64_t)h * Kt + i] = acc;
}

// D[h][i] in bf16: TPR = d / 8 consecutive lanes per (row, head), one
// 16-byte chunk of out and dout each (coalesced), then a fixed-order
// butterfly over the TPR lanes.
template <int TPR>
__global__ __launch_bounds__(256) void bwd_prep_bf16_kernel(const uint16_t* __restrict__ o,
                                                            const uint16_t* __restrict__ dout, int64_t Kt,
                                                            int Hq, float* __restrict__ D) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t idx = gid / TPR;  // (row, head)
  const int part = (int)(gid % TPR);
  const bool ok = idx < Kt * Hq;
  float acc = 0.0f;
  if (ok) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + idx * (8 * TPR) + 8 * part);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + idx * (8 * TPR) + 8 * part);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(__uint_as_float(av[j] << 16), __uint_as_float(bv[j] << 16), acc);
      acc = fmaf(__uint_as_float(av[j] & 0xffff0000u), __uint_as_float(bv[j] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (ok && part == 0) {
    const int64_t i = idx / Hq;
    D[(int64_t)(idx - i * Hq) * Kt + i] = acc;
  }
}

// ------------------------------------------------------------------- dq
template <int HD>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t qs, int64_t ks, int64_t vs, const float* __restrict__ bias, const float* __restrict__ gain,
    float tau, const int32_t* __restrict__ cu, int Hq, int group, int n_qt, int64_t Kt,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dv,
    uint16_t* __restrict__ dq, float* __restrict__ tau_part) {
  constexpr int KCH = HD / 8, NKS = HD / 16, NDB = HD / 32;
  constexpr int ROWN = KCH + 1, ROWT = KCH + 4;
  constexpr int ITEMS = kT * KCH / 256;  // 16-byte chunks per thread per tile (K, V each)
  __shared__ uint4 sK[kT * ROWN], sKT[kT * ROWT], sV[kT * ROWN];
  __shared__ __align__(16) float sS[kT];  // g_h log2(e) s_j of the tile's keys

  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5;
  // longest first; with several prompts the existing (prompt, tile) pairs
  // come first in the dispatch order (work_item)
  const long long rank = (long long)blockIdx.y + (long long)gridDim.y * blockIdx.z;
  int b = 0, tile = n_qt - 1 - (int)blockIdx.z;
  if (gridDim.y > 1) {
    work_item(cu, (int)gridDim.y, n_qt, 128, rank, lane, b, tile);
    b = __builtin_amdgcn_readfirstlane(b);
    tile = __builtin_amdgcn_readfirstlane(tile);
  }
  // the temperature partials are indexed by the slot, summed in slot order
  float* tp = tau_part + ((int64_t)h * gridDim.y * n_qt + rank) * 4;
  const int lo = cu[b];
  const int n = cu[b + 1] - lo;
  const int q0 = tile * 128;
  if (tile < 0 || q0 >= n) {
    if (tid < 4) tp[tid] = 0.0f;
    return;
  }
  const int kvh = h / group;
  const int qw = q0 + 32 * wave;
  const int my_q = qw + (lane & 31);
  const bool q_ok = my_q < n;
  const float c1 = tau * rsqrtf((float)HD) * kLog2eB;  // log2-domain scale of q.k
  const float gb = (bias && gain) ? gain[h] * kLog2eB : 0.0f;

  bf16x8 qf[NKS], gf[NKS];
  float lse2 = 0.0f, Di = 0.0f;
  {
    const uint16_t* qp = q + (int64_t)(lo + my_q) * qs + (int64_t)h * HD + 8 * G;
    const uint16_t* gp = dout + ((int64_t)(lo + my_q) * Hq + h) * HD + 8 * G;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      uint4 a = make_uint4(0, 0, 0, 0), c = a;
      if (q_ok) {
        a = *reinterpret_cast<const uint4*>(qp + 16 * s);
        c = *reinterpret_cast<const uint4*>(gp + 16 * s);
      }
      qf[s] = as_bf16x8(a);
      gf[s] = as_bf16x8(c);
    }
    if (q_ok) {
      lse2 = lse[(int64_t)h * Kt + lo + my_q] * kLog2eB;
      Di = Dv[(int64_t)h * Kt + lo + my_q];
    }
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  float tsum = 0.0f;

  const int kv_end = min(q0 + 128, n);
  const int n_kt = (kv_end + kT - 1) / kT;
  const uint16_t* kbase = k + (int64_t)lo * ks + (int64_t)kvh * HD;
  const uint16_t* vbase = v + (int64_t)lo * vs + (int64_t)kvh * HD;
  int offk[ITEMS], offv[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int id = tid + 256 * j;
    offk[j] = ((id / KCH) * (int)ks + (id % KCH) * 8) * 2;
    offv[j] = ((id / KCH) * (int)vs + (id % KCH) * 8) * 2;
  }
  uint4 rk[ITEMS], rv[ITEMS];
  float rs = 0.0f;
  auto prefetch = [&](int k0) __attribute__((always_inline)) {
    const int rows = __builtin_amdgcn_readfirstlane(max(min(n - k0, kT), 0));
    const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wave_uniform(kbase + (int64_t)k0 * ks), (short)0, rows * (int)ks * 2, kBufFlagsB);
    const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wave_uniform(vbase + (int64_t)k0 * vs), (short)0, rows * (int)vs * 2, kBufFlagsB);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      rk[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r1, offk[j], 0, 0));
      rv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r2, offv[j], 0, 0));
    }
    if (tid < kT) rs = (bias && k0 + tid < n) ? gb * bias[lo + k0 + tid] : 0.0f;
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int id = tid + 256 * j;
      sK[(id / KCH) * ROWN + id % KCH] = rk[j];
      sKT[(id / KCH) * ROWT + id % KCH] = rk[j];
      sV[(id / KCH) * ROWN + id % KCH] = rv[j];
    }
    if (tid < kT) sS[tid] = rs;
  };
  uint32_t kl = lds_addr(sK) + ((lane & 31) * ROWN + G) * 16, vl = lds_addr(sV) + ((lane & 31) * ROWN + G) * 16;
  uint32_t ktb = tr_lane_base<ROWT>(sKT, lane);
  asm volatile("" : "+v"(ktb), "+v"(kl), "+v"(vl));

  // Two workgroups share a CU: while one stages a tile (global loads, then
  // LDS writes, between two barriers), the other computes.
  for (int t = 0; t < n_kt; ++t) {
    prefetch(t * kT);
    __syncthreads();  // every wave is done with the previous tile
    stage();
    __syncthreads();
    const int k0 = t * kT;
    if (k0 > qw + 31 || qw >= n) continue;  // the tile lies past every row of this wave
    // the tile's two 32-key blocks one after the other (one S^T / dP^T
    // accumulator pair live at a time); dx^T of block kb goes straight into
    // the bf16 B operand of the 16-key steps 2 kb, 2 kb + 1 of dQ^T += K^T dx^T
    const bool full = (k0 + kT - 1 <= qw) && (qw + 32 <= n);  // no mask in this tile
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sa, sb;
#pragma unroll
      for (int i = 0; i < 16; ++i) sa[i] = sb[i] = 0.0f;
#pragma unroll
      for (int st = 0; st < NKS; ++st) {
        sa = mfma32x32x16(frag_at(kl, (32 * kb * ROWN + 2 * st) * 16), qf[st], sa);
        sb = mfma32x32x16(frag_at(vl, (32 * kb * ROWN + 2 * st) * 16), gf[st], sb);
      }
      bf16x8 pb[2];
      auto elems = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int key0 = kb * 32 + acc_row(4 * r4, lane);  // registers 4 r4 .. +3: keys key0 .. key0 + 3
          const float4 B4 = *reinterpret_cast<const float4*>(sS + key0);
          const float Br[4] = {B4.x, B4.y, B4.z, B4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 4 * r4 + j;
            float p = __builtin_amdgcn_exp2f(fmaf(sa[i], c1, Br[j]) - lse2);
            if constexpr (decltype(masked)::value) p = (q_ok & (k0 + key0 + j <= my_q)) ? p : 0.0f;
            const float dxv = p * (sb[i] - Di);
            tsum = fmaf(dxv, sa[i], tsum);
            pb[i >> 3][i & 7] = (__bf16)dxv;
          }
        }
      };
      if (full)
        elems(std::false_type{});
      else
        elems(std::true_type{});
#pragma unroll
      for (int r16 = 0; r16 < 2; ++r16)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          acc[db] = mfma32x32x16(frag_tr<ROWT>(ktb, 2 * kb + r16, db), pb[r16], acc[db]);
    }
  }
  const float tw = wave_sum(tsum);
  if (lane == 0) tp[wave] = tw;
  const float scale = tau * rsqrtf((float)HD);
  uint16_t* dp_out = dq + ((int64_t)(lo + min(my_q, n - 1)) * Hq + h) * HD;  // rows past the prompt store nothing
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_bf16_rows(dp_out + 32 * db, acc[db], scale, G, q_ok);
}

// ----------------------------------------------------------------- dk, dv
// Two passes over the same query tiles, each light enough for two workgroups
// per CU: DK = false accumulates dV^T += dO^T P (it needs only S); DK = true
// accumulates dK^T += Q^T dx and the column sums of dx (it needs S and dP).
// Recomputing S in both costs one product in five and halves the registers
// each pass holds.  One workgroup per query head: a key tile's longest chain
// is then one head's query tiles, not the whole group's, and the grid has
// Hq (not Hkv) workgroups per key tile.  With a group of several heads each
// writes its fp32 sums to part [Hq][Kt][HD] and bwd_group_sum adds the
// group's in head order; with one head per group the workgroup stores the
// bf16 rows itself (part == nullptr).
template <int HD, bool DK>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t qs, int64_t ks, int64_t vs, const float* __restrict__ bias, const float* __restrict__ gain,
    float tau, const int32_t* __restrict__ cu, int Hq, int Hkv, int group, int64_t Kt,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dv,
    uint16_t* __restrict__ dkv, float* __restrict__ part, float* __restrict__ colsum) {
  constexpr int KCH = HD / 8, NKS = HD / 16, NDB = HD / 32;
  constexpr int ROWN = KCH + 1, ROWT = KCH + 4;
  constexpr int ITEMS = kT * KCH / 256;
  // DK: sQ (normal), sO (normal), sQT (transposing reads); dV: sQ, sOT
  __shared__ uint4 sm[DK ? kT * (2 * ROWN + ROWT) : kT * (ROWN + ROWT)];
  __shared__ __align__(16) float sL[kT];
  __shared__ __align__(16) float sD[DK ? kT : 4];
  uint4* const sQ = sm;
  uint4* const sX = sm + kT * ROWN;  // sO (DK) or sOT (dV)
  uint4* const sQT = sm + 2 * kT * ROWN;

  const int h = blockIdx.x;
  const int kvh = h / group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the first key tiles see the most queries: launched first.  Key tile t
  // of a prompt with n_b tiles sees n_b - t query-tile steps, so with
  // several prompts work_item's order (index descending) over u = n_b - 1 -
  // t puts the existing pairs first, most work first.
  int b = 0, tile = blockIdx.z;
  if (gridDim.y > 1) {
    int u = 0;
    work_item(cu, (int)gridDim.y, (int)gridDim.z, 128, (long long)blockIdx.y + (long long)gridDim.y * blockIdx.z,
              lane, b, u);
    b = __builtin_amdgcn_readfirstlane(b);
    u = __builtin_amdgcn_readfirstlane(u);
    if (u < 0) return;
    tile = tiles_of(cu, b, 128) - 1 - u;
  }
  const int lo = cu[b];
  const int n = cu[b + 1] - lo;
  const int k0w = tile * 128;
  if (k0w >= n) return;
  const int G = lane >> 5;
  const int kw = k0w + 32 * wave;
  const int my_k = kw + (lane & 31);
  const bool k_ok = my_k < n;
  const float c1 = tau * rsqrtf((float)HD) * kLog2eB;

  bf16x8 kf[NKS], vf[DK ? NKS : 1];
  {
    const uint16_t* kp = k + (int64_t)(lo + my_k) * ks + (int64_t)kvh * HD + 8 * G;
    const uint16_t* vp = v + (int64_t)(lo + my_k) * vs + (int64_t)kvh * HD + 8 * G;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      uint4 a = make_uint4(0, 0, 0, 0);
      if (k_ok) a = *reinterpret_cast<const uint4*>(kp + 16 * s);
      kf[s] = as_bf16x8(a);
      if constexpr (DK) {
        uint4 c = make_uint4(0, 0, 0, 0);
        if (k_ok) c = *reinterpret_cast<const uint4*>(vp + 16 * s);
        vf[s] = as_bf16x8(c);
      }
    }
  }
  const float sj = (bias && k_ok) ? bias[lo + my_k] : 0.0f;
  const float bj = (bias && gain) ? gain[h] * kLog2eB * sj : 0.0f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;

  const int t_first = k0w / kT;
  const int n_qtl = (n + kT - 1) / kT;
  int offq[ITEMS], offo[ITEMS];
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int id = tid + 256 * j;
    offq[j] = ((id / KCH) * (int)qs + (id % KCH) * 8) * 2;
    offo[j] = ((id / KCH) * Hq * HD + (id % KCH) * 8) * 2;
  }
  uint4 rq[ITEMS], ro[ITEMS];
  float rl = 0.0f, rd = 0.0f;
  auto prefetch = [&](int h, int i0) __attribute__((always_inline)) {
    const int rows = __builtin_amdgcn_readfirstlane(max(min(n - i0, kT), 0));
    const __amdgpu_buffer_rsrc_t r1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wave_uniform(q + (int64_t)(lo + i0) * qs + (int64_t)h * HD), (short)0, rows * (int)qs * 2, kBufFlagsB);
    const __amdgpu_buffer_rsrc_t r2 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wave_uniform(dout + ((int64_t)(lo + i0) * Hq + h) * HD), (short)0, rows * Hq * HD * 2, kBufFlagsB);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      rq[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r1, offq[j], 0, 0));
      ro[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r2, offo[j], 0, 0));
    }
    if (tid < kT) {
      const bool ok = i0 + tid < n;
      rl = ok ? lse[(int64_t)h * Kt + lo + i0 + tid] * kLog2eB : 0.0f;
      if constexpr (DK) rd = ok ? Dv[(int64_t)h * Kt + lo + i0 + tid] : 0.0f;
    }
  };
  auto stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int id = tid + 256 * j;
      sQ[(id / KCH) * ROWN + id % KCH] = rq[j];
      if constexpr (DK) {
        sQT[(id / KCH) * ROWT + id % KCH] = rq[j];
        sX[(id / KCH) * ROWN + id % KCH] = ro[j];
      } else {
        sX[(id / KCH) * ROWT + id % KCH] = ro[j];
      }
    }
    if (tid < kT) {
      sL[tid] = rl;
      if constexpr (DK) sD[tid] = rd;
    }
  };
  uint32_t ql = lds_addr(sQ) + ((lane & 31) * ROWN + G) * 16, ol = lds_addr(sX) + ((lane & 31) * ROWN + G) * 16;
  // transposing reads: of Q for dK, of dO for dV
  uint32_t trb = DK ? tr_lane_base<ROWT>(sQT, lane) : tr_lane_base<ROWT>(sX, lane);
  asm volatile("" : "+v"(trb), "+v"(ql));
  if constexpr (DK) asm volatile("" : "+v"(ol));

  float csum = 0.0f;
  // last query tile first: every workgroup starts on the same tiles at the
  // same time and walks down in near lockstep, so each staged Q / dO tile
  // is fetched from memory once per L2 and reused by the others
  for (int t = n_qtl - 1; t >= t_first; --t) {
    const int i0 = t * kT;
    prefetch(h, i0);
    __syncthreads();  // every wave is done with the previous tile
    stage();
    __syncthreads();
    const bool active = (kw < n) && (i0 + kT - 1 >= kw);  // some query of the tile sees a key of the wave
    // every query of the tile sees every key of the wave, all of them valid
    const bool full = (i0 >= kw + 31) && (i0 + kT <= n) && (kw + 32 <= n);
    if (active) {
      // the tile's two 32-query halves one after the other (one S / dP
      // accumulator pair live at a time): P (dV) or dx (DK) of half qb is
      // the B operand of the 16-row steps 2 qb, 2 qb + 1
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sa, sb;
#pragma unroll
        for (int i = 0; i < 16; ++i) sa[i] = sb[i] = 0.0f;
#pragma unroll
        for (int st = 0; st < NKS; ++st) {
          sa = mfma32x32x16(frag_at(ql, (32 * qb * ROWN + 2 * st) * 16), kf[st], sa);
          if constexpr (DK) sb = mfma32x32x16(frag_at(ol, (32 * qb * ROWN + 2 * st) * 16), vf[st], sb);
        }
        // registers 4 r4 .. 4 r4 + 3 hold rows qr0 .. qr0 + 3: their lse
        // (and D) in one 16-byte LDS read; the exponent is evaluated for
        // every element and masked by a select (no branch around the read)
        bf16x8 xb[2];
        auto elems = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int qr0 = qb * 32 + acc_row(4 * r4, lane);
            const float4 L4 = *reinterpret_cast<const float4*>(sL + qr0);
            float4 D4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if constexpr (DK) D4 = *reinterpret_cast<const float4*>(sD + qr0);
            const float Lr[4] = {L4.x, L4.y, L4.z, L4.w}, Dr[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 4 * r4 + j;
              float p = __builtin_amdgcn_exp2f(fmaf(sa[i], c1, bj) - Lr[j]);
              if constexpr (decltype(masked)::value) {
                const int qi = i0 + qr0 + j;
                p = (k_ok & (qi >= my_k) & (qi < n)) ? p : 0.0f;
              }
              float x = p;
              if constexpr (DK) {
                x = p * (sb[i] - Dr[j]);
                csum += x;
              }
              xb[i >> 3][i & 7] = (__bf16)x;
            }
          }
        };
        if (full)
          elems(std::false_type{});
        else
          elems(std::true_type{});
#pragma unroll
        for (int r16 = 0; r16 < 2; ++r16)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = mfma32x32x16(frag_tr<ROWT>(trb, 2 * qb + r16, db), xb[r16], acc[db]);
      }
    }
  }
  if constexpr (DK) {
    const float c = pair_sum(csum);
    if (k_ok && G == 0) colsum[(int64_t)h * Kt + lo + my_k] = c;
  }
  if (part) {
    if (!k_ok) return;
    float* pp = part + ((int64_t)h * Kt + lo + my_k) * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(pp + 32 * db + 8 * g4 + 4 * G) =
            make_float4(acc[db][4 * g4], acc[db][4 * g4 + 1], acc[db][4 * g4 + 2], acc[db][4 * g4 + 3]);
    return;
  }
  const float scale = DK ? tau * rsqrtf((float)HD) : 1.0f;
  uint16_t* op = dkv + ((int64_t)(lo + min(my_k, n - 1)) * Hkv + kvh) * HD;  // rows past the prompt store nothing
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_bf16_rows(op + 32 * db, acc[db], scale, G, k_ok);
}

// out[r][kvh][e] = bf16(mul * sum_(hh < group) part[kvh group + hh][r][e]),
// heads in order; 4 elements per thread.
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float* __restrict__ part, int64_t Kt, int Hkv,
                                                            int group, int d, float mul, uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, kvh, 4-element chunk)
  const int nc = d / 4;
  if (idx >= Kt * Hkv * nc) return;
  const int64_t r = idx / ((int64_t)Hkv * nc);
  const int rem = (int)(idx - r * Hkv * nc);
  const int kvh = rem / nc, c = rem % nc;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int hh = 0; hh < group; ++hh) {
    const float4 x = *reinterpret_cast<const float4*>(part + ((int64_t)(kvh * group + hh) * Kt + r) * d + 4 * c);
    a.x += x.x;
    a.y += x.y;
    a.z += x.z;
    a.w += x.w;
  }
  const unsigned w0 = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)(a.x * mul)) |
                      ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)(a.y * mul)) << 16);
  const unsigned w1 = (unsigned)__builtin_bit_cast(uint16_t, (__bf16)(a.z * mul)) |
                      ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)(a.w * mul)) << 16);
  *reinterpret_cast<uint2*>(out + ((r * Hkv + kvh) * d + 4 * c)) = make_uint2(w0, w1);
}


// ------------------------------------------------------------- fp32 paths
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    int64_t qs, int64_t ks, int64_t vs, const float* __restrict__ bias, const float* __restrict__ gain,
    float tau, const int32_t* __restrict__ cu, int B, int Hq, int group, int d, int64_t Kt,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dv,
    float* __restrict__ dq, float* __restrict__ tau_part) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= Kt * Hq) return;
  const int64_t i = idx / Hq;
  const int h = (int)(idx - i * Hq);
  int b = 0;
  while (b + 1 < B && cu[b + 1] <= i) ++b;
  const int64_t lo = cu[b];
  const int kvh = h / group;
  const float sc = tau / sqrtf((float)d);
  const float g = (bias && gain) ? gain[h] : 0.0f;
  const float L = lse[(int64_t)h * Kt + i], Di = Dv[(int64_t)h * Kt + i];
  const float* qi = q + i * qs + (int64_t)h * d;
  const float* gi = dout + (i * Hq + h) * d;
  float acc[128];
  for (int e = 0; e < d; ++e) acc[e] = 0.0f;
  float ts = 0.0f;
  for (int64_t j = lo; j <= i; ++j) {
    const float* kj = k + j * ks + (int64_t)kvh * d;
    const float* vj = v + j * vs + (int64_t)kvh * d;
    float qk = 0.0f, dp = 0.0f;
    for (int e = 0; e < d; ++e) {
      qk = fmaf(qi[e], kj[e], qk);
      dp = fmaf(gi[e], vj[e], dp);
    }
    const float p = expf(sc * qk + (g != 0.0f ? g * bias[j] : 0.0f) - L);
    const float dx = p * (dp - Di);
    ts = fmaf(dx, qk, ts);
    for (int e = 0; e < d; ++e) acc[e] = fmaf(dx, kj[e], acc[e]);
  }
  float* out = dq + (i * Hq + h) * d;
  for (int e = 0; e < d; ++e) out[e] = sc * acc[e];
  tau_part[idx] = ts;
}

__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    int64_t qs, int64_t ks, int64_t vs, const float* __restrict__ bias, const float* __restrict__ gain,
    float tau, const int32_t* __restrict__ cu, int B, int Hq, int Hkv, int group, int d, int64_t Kt,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ Dv,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ colsum) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= Kt * Hkv) return;
  const int64_t j = idx / Hkv;
  const int kvh = (int)(idx - j * Hkv);
  int b = 0;
  while (b + 1 < B && cu[b + 1] <= j) ++b;
  const int64_t hi = cu[b + 1];
  const float sc = tau / sqrtf((float)d);
  const float* kj = k + j * ks + (int64_t)kvh * d;
  const float* vj = v + j * vs + (int64_t)kvh * d;
  float ak[128], av[128];
  for (int e = 0; e < d; ++e) ak[e] = av[e] = 0.0f;
  for (int hh = 0; hh < group; ++hh) {
    const int h = kvh * group + hh;
    const float g = (bias && gain) ? gain[h] : 0.0f;
    float cs = 0.0f;
    for (int64_t i = j; i < hi; ++i) {
      const float* qi = q + i * qs + (int64_t)h * d;
      const float* gi = dout + (i * Hq + h) * d;
      float qk = 0.0f, dp = 0.0f;
      for (int e = 0; e < d; ++e) {
        qk = fmaf(qi[e], kj[e], qk);
        dp = fmaf(gi[e], vj[e], dp);
      }
      const float p = expf(sc * qk + (g != 0.0f ? g * bias[j] : 0.0f) - lse[(int64_t)h * Kt + i]);
      const float dx = p * (dp - Dv[(int64_t)h * Kt + i]);
      cs += dx;
      for (int e = 0; e < d; ++e) {
        ak[e] = fmaf(dx, qi[e], ak[e]);
        av[e] = fmaf(p, gi[e], av[e]);
      }
    }
    colsum[(int64_t)h * Kt + j] = cs;
  }
  float* ko = dk + (j * Hkv + kvh) * d;
  float* vo = dv + (j * Hkv + kvh) * d;
  for (int e = 0; e < d; ++e) {
    ko[e] = sc * ak[e];
    vo[e] = av[e];
  }
}

// ------------------------------------------------------------- finalize
// ds_j = sum_h g_h c_hj (h in order), one thread per key.
__global__ __launch_bounds__(256) void bwd_ds_kernel(const float* __restrict__ colsum, const float* __restrict__ gain,
                                                     int Hq, int64_t Kt, float* __restrict__ ds) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= Kt) return;
  float acc = 0.0f;
  for (int h = 0; h < Hq; ++h) acc = fmaf(gain[h], colsum[(int64_t)h * Kt + j], acc);
  ds[j] = acc;
}

// Workgroup h < Hq: dg_h = sum_j s_j c_hj; workgroup Hq: dtau = sum of the
// partials / sqrt(d).  Strided per-thread sums, then a fixed tree in LDS.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ colsum, const float* __restrict__ bias,
                                                         int Hq, int64_t Kt, const float* __restrict__ tau_part,
                                                         int64_t n_part, float inv_sqrt_d, float* __restrict__ dg,
                                                         float* __restrict__ dtau) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  float acc = 0.0f;
  if (h < Hq) {
    if (dg) for (int64_t j = tid; j < Kt; j += 256) acc = fmaf(bias[j], colsum[(int64_t)h * Kt + j], acc);
  } else {
    for (int64_t j = tid; j < n_part; j += 256) acc += tau_part[j];
  }
  red[tid] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) {
    if (h < Hq) {
      if (dg) dg[h] = red[0];
    } else if (dtau) {
      *dtau = red[0] * inv_sqrt_d;
    }
  }
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// D, column sums, dtau partials; bf16 with several heads per KV head: the
// per-head fp32 dK and dV sums
size_t attn_bwd_workspace_bytes(int B, int64_t Kt, int Hq, int Hkv, int d, int elem_bytes, int max_len) {
  const int64_t n_qt = ((int64_t)max_len + 127) / 128;
  const int64_t n_part = std::max<int64_t>((int64_t)Hq * B * n_qt * 4, Kt * Hq);
  size_t bytes = 2 * align256((size_t)Hq * Kt * 4) + align256((size_t)n_part * 4);
  if (elem_bytes == 2 && Hq != Hkv) bytes += 2 * align256((size_t)Hq * Kt * d * 4);
  return bytes;
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                           const float* bias, const float* gain, float tau, const int32_t* cu, int B,
                           int max_len, int64_t Kt, int Hq, int Hkv, int d, int elem_bytes, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, float* ds,
                           float* dg, float* dtau, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  float* Dv = reinterpret_cast<float*>(w);
  float* colsum = reinterpret_cast<float*>(w + align256((size_t)Hq * Kt * 4));
  float* tpart = reinterpret_cast<float*>(w + 2 * align256((size_t)Hq * Kt * 4));
  const int group = Hq / Hkv;
  const size_t head_off = 2 * align256((size_t)Hq * Kt * 4) +
                          align256((size_t)std::max<int64_t>((int64_t)Hq * B * ((max_len + 127) / 128) * 4, Kt * Hq) * 4);
  float* part_k = group > 1 ? reinterpret_cast<float*>(w + head_off) : nullptr;
  float* part_v = group > 1 ? reinterpret_cast<float*>(w + head_off + align256((size_t)Hq * Kt * d * 4)) : nullptr;
  const int64_t rows = Kt * Hq;
  const bool has_bias = bias && gain;
  if (elem_bytes == 2 && d == 128)
    hipLaunchKernelGGL(bwd_prep_bf16_kernel<16>, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), Kt, Hq, Dv);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(bwd_prep_bf16_kernel<8>, dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(out), static_cast<const uint16_t*>(dout), Kt, Hq, Dv);
  else
    hipLaunchKernelGGL(bwd_prep_f32_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s,
                       static_cast<const float*>(out), static_cast<const float*>(dout), Kt, Hq, d, Dv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t n_part;
  if (elem_bytes == 2) {
    const int n_qt = (max_len + 127) / 128;
    n_part = (int64_t)Hq * B * n_qt * 4;
    const auto* qp = static_cast<const uint16_t*>(q);
    const auto* kp = static_cast<const uint16_t*>(k);
    const auto* vp = static_cast<const uint16_t*>(v);
    const auto* gp = static_cast<const uint16_t*>(dout);
    const dim3 gq((unsigned)Hq, (unsigned)B, (unsigned)n_qt);
    const dim3 gk((unsigned)Hq, (unsigned)B, (unsigned)n_qt);
    if (d == 128) {
      hipLaunchKernelGGL(bwd_dq_kernel<128>, gq, dim3(256), 0, s, qp, kp, vp, qs, ks, vs, bias, gain, tau, cu, Hq,
                         group, n_qt, Kt, gp, lse, Dv, static_cast<uint16_t*>(dq), tpart);
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), gk, dim3(256), 0, s, qp, kp, vp, qs, ks, vs, bias, gain, tau,
                         cu, Hq, Hkv, group, Kt, gp, lse, Dv, static_cast<uint16_t*>(dv), part_v, colsum);
      hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), gk, dim3(256), 0, s, qp, kp, vp, qs, ks, vs, bias, gain, tau,
                         cu, Hq, Hkv, group, Kt, gp, lse, Dv, static_cast<uint16_t*>(dk), part_k, colsum);
    } else {
      hipLaunchKernelGGL(bwd_dq_kernel<64>, gq, dim3(256), 0, s, qp, kp, vp, qs, ks, vs, bias, gain, tau, cu, Hq,
                         group, n_qt, Kt, gp, lse, Dv, static_cast<uint16_t*>(dq), tpart);
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), gk, dim3(256), 0, s, qp, kp, vp, qs, ks, vs, bias, gain, tau,
                         cu, Hq, Hkv, group, Kt, gp, lse, Dv, static_cast<uint16_t*>(dv), part_v, colsum);
      hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), gk, dim3(256), 0, s, qp, kp, vp, qs, ks, vs, bias, gain, tau,
                         cu, Hq, Hkv, group, Kt, gp, lse, Dv, static_cast<uint16_t*>(dk), part_k, colsum);
    }
    if (group > 1) {
      const unsigned nb = (unsigned)((Kt * Hkv * (d / 4) + 255) / 256);
      hipLaunchKernelGGL(bwd_group_sum_kernel, dim3(nb), dim3(256), 0, s, part_v, Kt, Hkv, group, d, 1.0f,
                         static_cast<uint16_t*>(dv));
      hipLaunchKernelGGL(bwd_group_sum_kernel, dim3(nb), dim3(256), 0, s, part_k, Kt, Hkv, group, d,
                         tau / sqrtf((float)d), static_cast<uint16_t*>(dk));
    }
  } else {
    n_part = rows;
    const auto* qp = static_cast<const float*>(q);
    const auto* kp = static_cast<const float*>(k);
    const auto* vp = static_cast<const float*>(v);
    const auto* gp = static_cast<const float*>(dout);
    hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, qp, kp, vp, qs, ks,
                       vs, bias, gain, tau, cu, B, Hq, group, d, Kt, gp, lse, Dv, static_cast<float*>(dq), tpart);
    hipLaunchKernelGGL(bwd_dkdv_f32_kernel, dim3((unsigned)((Kt * Hkv + 255) / 256)), dim3(256), 0, s, qp, kp, vp,
                       qs, ks, vs, bias, gain, tau, cu, B, Hq, Hkv, group, d, Kt, gp, lse, Dv,
                       static_cast<float*>(dk), static_cast<float*>(dv), colsum);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // without the bias term ds and dg are zero (filled by a kernel, so that a
  // captured graph holds no memset node)
  if (ds) {
    if (has_bias)
      hipLaunchKernelGGL(bwd_ds_kernel, dim3((unsigned)((Kt + 255) / 256)), dim3(256), 0, s, colsum, gain, Hq, Kt, ds);
    else
      hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((Kt + 255) / 256)), dim3(256), 0, s, ds, Kt);
  }
  if (dg && !has_bias)
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((Hq + 255) / 256)), dim3(256), 0, s, dg, (int64_t)Hq);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)Hq + 1), dim3(256), 0, s, colsum, bias, Hq, Kt, tpart, n_part,
                     1.0f / sqrtf((float)d), has_bias ? dg : nullptr, dtau);
  return hipGetLastError();
}

}  // namespace tg

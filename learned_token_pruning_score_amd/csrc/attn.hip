// Token-gated causal GQA attention over the kept tokens (TokenGate article,
// section "What is token-gated attention?": each kept token's score becomes
// an additive bias on the attention logits above the gate, with a learnable
// per-head gain and a learnable temperature):
//     x_ij = tau * q_i . k_j / sqrt(d) + g_h * s_j,   j <= i within a prompt
//     o_i  = softmax_j(x_ij) v_j,  lse_i = ln sum_j exp(x_ij)
//
// bf16 path (gfx950 MFMA, fp32 accumulation), one workgroup of 4 waves per
// (query head, prompt, 128-row query tile); wave w owns rows 32w..32w+31.
//  * Scores are formed transposed, S^T = K Q^T, with the 32x32x16 MFMA: lane
//    l then holds 32 keys of query row (l & 31) per 64-key tile, so the
//    softmax max and sum are lane-local plus one exchange with lane l ^ 32.
//  * The bias and temperature fold into one FMA in the log2 domain:
//    y = acc * (tau log2e / sqrt(d)) + (g_h log2e) s_j; p = exp2(y - m).
//  * P^T stays in registers: the accumulator layout of S^T is exactly the B
//    operand layout of O^T += V^T P^T once keys are relabelled (within each
//    16-key MFMA step, lane half G holds keys 4G..4G+3 and 8+4G..8+4G+3); V
//    stays row-major in LDS and a transposing LDS read delivers those keys.
//  * K rows and V^T rows are padded in LDS (odd multiples of the read
//    width) so fragment reads of 32 rows spread over the banks.
//  * Two LDS stages: the next tile's global loads are issued before the
//    current tile's MFMAs and written to the other stage after them.
//  * Causal masking only on tiles that cross the wave's diagonal; tiles are
//    launched longest-first (tile index is the slowest grid dimension,
//    reversed); the heads of one GQA group land on the same XCD.
// fp32 path: one thread per (row, head), online softmax on vector ALUs.
#include <math.h>

#include <type_traits>

#include "tg_common.h"

namespace tg {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBK = 64;   // keys per tile
constexpr float kRescale = 8.0f;
// Fourth word of a raw buffer descriptor (32-bit data format, no swizzle):
// accesses at or past num_records read as zero.
constexpr int kBufFlags = 0x00020000;  // lazy-rescale threshold on the running max (log2 units)
#ifndef TG_ATTN_WAVES
#define TG_ATTN_WAVES 8   // waves per workgroup; 32 query rows each
#endif

// LDS rows are padded so that a fragment read of 32 consecutive rows at one
// column spreads over the banks, and every per-step offset is a constant:
// a K row is HD*2 + 16 bytes (an odd number of 16-byte units), a V^T row is
// 64 keys * 2 + 8 = 136 bytes (an odd number of 8-byte units).

__device__ __forceinline__ unsigned elem16(const uint4& v, int e) {
  const unsigned w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t qs, int64_t ks, int64_t vs,
    const float* __restrict__ bias, const float* __restrict__ gain, float qk_scale,
    const int32_t* __restrict__ cu, int Hq, int group, int head_swizzle, int n_qtiles,
    int64_t Kt, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = NW * 64;
  constexpr int BQ = 32 * NW;       // query rows per workgroup
  constexpr int KCH = HD / 8;       // 16-byte chunks per K row
  constexpr int NKS = HD / 16;      // MFMA k-steps over the head dim
  constexpr int NDB = HD / 32;      // 32-row blocks of O^T
  constexpr int K_ITEMS = kBK * KCH;
  constexpr int K_PER_T = (K_ITEMS + NT - 1) / NT;
  constexpr int V_ITEMS = kBK * KCH;  // 16-byte chunks of a V tile
  constexpr int V_PER_T = (V_ITEMS + NT - 1) / NT;
  constexpr int KROW = KCH + 1;     // 16-byte units per padded K row
  constexpr int VROW = KCH + 2;     // 16-byte units per padded V row (HD*2 + 32 bytes)
  // Two LDS stages: the next tile is written while the current one is read.
  __shared__ uint4 sK[2][kBK * KROW];
  __shared__ uint4 sV[2][kBK * VROW];
  __shared__ uint32_t sB[2][kBK];  // per key: bias / scale as a bf16 (hi, lo) pair

  const int x = blockIdx.x;
  const int h = head_swizzle ? (x % 8) * (Hq / 8) + x / 8 : x;
  const int b = blockIdx.y;
  const int tile = n_qtiles - 1 - (int)blockIdx.z;
  const int lo = cu[b];
  const int n = cu[b + 1] - lo;
  const int q0 = tile * BQ;
  if (q0 >= n) return;
  const int kvh = h / group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int G = lane >> 5;
  const int qw = q0 + wave * 32;
  const int my_q = qw + (lane & 31);
  // The key bias enters the score MFMA as one more k-step: K gains the
  // columns (c_hi, c_lo) with c_hi + c_lo = g_h log2e s_j / scale (two bf16
  // parts, exact to about 2^-16 of c) and Q gains the columns (1, 1), so the
  // accumulator holds q.k + c and the logit is scale * acc.  The softmax then
  // needs one FMA per score.  Requires scale > 0 (checked on the host).
  const bool has_bias = (bias != nullptr) && (gain != nullptr);
  const float cmul = has_bias ? gain[h] * kLog2e / qk_scale : 0.0f;
  const bf16x8 q_one = as_bf16x8(make_uint4(G == 0 ? 0x3F803F80u : 0u, 0u, 0u, 0u));
  const float rs_thr = kRescale / qk_scale;  // rescale threshold in accumulator units

  bf16x8 qf[NKS];
  {
    const uint16_t* qp = q + (int64_t)(lo + my_q) * qs + (int64_t)h * HD + 8 * G;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (my_q < n) u = *reinterpret_cast<const uint4*>(qp + 16 * s);
      qf[s] = as_bf16x8(u);
    }
  }
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m_run = -INFINITY;  // running max of the accumulator (q.k + c)
  float nms = 0.0f;         // -m_run * scale
  float l_run = 0.0f;

  const int kv_end = min(q0 + BQ, n);
  const int n_kt = (kv_end + kBK - 1) / kBK;
  const bool wave_active = qw < n;
  const int n_kt_w = wave_active ? min(qw + 31, n - 1) / kBK + 1 : 0;
  const uint16_t* kbase = k + (int64_t)lo * ks + (int64_t)kvh * HD;
  const uint16_t* vbase = v + (int64_t)lo * vs + (int64_t)kvh * HD;

  static_assert(K_ITEMS % NT == 0 && V_ITEMS % NT == 0, "tile split");
  // Buffer-resource loads: the descriptor of each tile starts at its first
  // key and ends at the prompt's last key (or 64 keys on), so rows past the
  // prompt read as zero without a branch.  Such keys only occur in a tile
  // that crosses the causal diagonal of every wave reading it, where they
  // are masked.  Per-thread byte offsets are loop-invariant.
  int k_off[K_PER_T];
#pragma unroll
  for (int j = 0; j < K_PER_T; ++j) {
    const int id = tid + j * NT;
    k_off[j] = ((id / KCH) * (int)ks + (id % KCH) * 8) * 2;
  }
  int v_off[V_PER_T];
#pragma unroll
  for (int j = 0; j < V_PER_T; ++j) {
    const int id = tid + j * NT;
    v_off[j] = ((id / KCH) * (int)vs + (id % KCH) * 8) * 2;
  }
  const float* bias_p = bias ? bias + lo : nullptr;

  uint4 kreg[K_PER_T];
  uint4 vreg[V_PER_T];
  float breg = 0.0f;
  auto prefetch = [&](int k0) {
    const int rows = min(n - k0, kBK);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (int64_t)k0 * ks), (short)0, rows * (int)ks * 2, kBufFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (int64_t)k0 * vs), (short)0, rows * (int)vs * 2, kBufFlags);
#pragma unroll
    for (int j = 0; j < K_PER_T; ++j)
      kreg[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_off[j], 0, 0));
#pragma unroll
    for (int j = 0; j < V_PER_T; ++j)
      vreg[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, v_off[j], 0, 0));
    if (bias_p != nullptr) {
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(bias_p + k0), (short)0, rows * 4, kBufFlags);
      breg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (tid & (kBK - 1)) * 4, 0, 0));
    }
  };
  // Registers -> LDS stage `buf`: K and V rows copied as they are (padded
  // rows), bias pre-scaled.
  auto stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < K_PER_T; ++j) {
      const int id = tid + j * NT;
      sK[buf][(id / KCH) * KROW + (id % KCH)] = kreg[j];
    }
#pragma unroll
    for (int j = 0; j < V_PER_T; ++j) {
      const int id = tid + j * NT;
      sV[buf][(id / KCH) * VROW + (id % KCH)] = vreg[j];
    }
    if (tid < kBK) {
      const float c = breg * cmul;
      const __bf16 c_hi = (__bf16)c;
      const __bf16 c_lo = (__bf16)(c - (float)c_hi);
      sB[buf][tid] = (uint32_t)__builtin_bit_cast(uint16_t, c_hi) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, c_lo) << 16);
    }
  };

  // One 64-key tile for this wave's 32 rows.  MASK: the tile crosses the
  // wave's causal diagonal.  The running max is only moved when a row's max
  // grows by more than kRescale (log2 units): until then p <= 2^kRescale,
  // harmless in fp32 and bf16, and the O/l rescale is skipped.
  auto tile_step = [&](int buf, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // All fragment reads of the tile are issued before its MFMAs, so their
    // LDS latency overlaps, and the two 32-key MFMA chains are interleaved
    // so neither waits on its own previous result.
    f32x16 s[2];
    uint4 cb[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      cb[kb] = make_uint4((has_bias && G == 0) ? sB[buf][kb * 32 + (lane & 31)] : 0u, 0u, 0u, 0u);
    uint4 kf[2][NKS];
#pragma unroll
    for (int st = 0; st < NKS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kf[kb][st] = sK[buf][(kb * 32 + (lane & 31)) * KROW + 2 * st + G];
    __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the MFMAs
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
    for (int st = 0; st < NKS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(as_bf16x8(kf[kb][st]), qf[st], s[kb]);
    if (has_bias) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(as_bf16x8(cb[kb]), q_one, s[kb]);
    }
    // V^T fragments of the value product, read now so their LDS latency
    // overlaps the softmax below.  A transposing LDS read
    // (ds_read_b64_tr_b16) turns the row-major V tile into the MFMA operand:
    // within each 16-lane group, lane i receives element i % 4 of the 8-byte
    // chunks addressed by lanes 4j + i / 4 (j = 0..3).  Lane s of group g
    // therefore addresses key row 4 (g / 2) + s / 4 and columns
    // 16 (g % 2) + 4 (s % 4) .. +3 of a 16-key step, and lane l receives keys
    // 4G..4G+3 (then +8..+11) of head-dim row l % 32 of the block.
    bf16x8 vf[NDB][4];
    {
      const int gi = lane & 15, g = lane >> 4;
      const char* vb = reinterpret_cast<const char*>(&sV[buf][0]) +
                       (4 * (g >> 1) + (gi >> 2)) * (VROW * 16) + (16 * (g & 1) + 4 * (gi & 3)) * 2;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kh = 0; kh < 4; ++kh) {  // (kb, hh) = (kh / 2, kh % 2): keys kb*32 + 16hh ..
          const char* p0 = vb + ((kh >> 1) * 32 + 16 * (kh & 1)) * (VROW * 16) + db * 64;
          typedef short s4 __attribute__((ext_vector_type(4)));
          const s4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s4*)(p0));
          const s4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s4*)(p0 + 8 * (VROW * 16)));
          vf[db][kh] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (MASK) {
          const int key = kb * 32 + acc_row(i, lane);
          if ((k0 + key) > my_q) s[kb][i] = -INFINITY;
        }
        mx = fmaxf(mx, s[kb][i]);
      }
    mx = pair_max(mx);
    if (__any(mx > m_run + rs_thr)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * qk_scale);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_run = m_new;
      nms = -m_new * qk_scale;
    }
    float psum = 0.0f;  // fp32 row sum (keeps lse exact to fp32 rounding)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], qk_scale, nms));
        psum += s[kb][i];
      }
    l_run += psum;

    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[kb][hh][j] = (__bf16)s[kb][8 * hh + j];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kh = 0; kh < 4; ++kh)
        o[db] = mfma32x32x16(vf[db][kh], pb[kh >> 1][kh & 1], o[db]);
  };

  // n_kt >= 1 here (q0 < n).  The unconditional first stage also retires the
  // Q loads on every path into the loop.
  prefetch(0);
  stage(0);
  __syncthreads();

  // Every wave runs n_kt iterations (one barrier each) but computes only on
  // the tiles its rows see: unmasked tiles, then the one tile crossing its
  // diagonal, then staging-only iterations.  Three straight loops keep the
  // accumulators in place (no merge of differently computed values).
  auto iteration = [&](int kt, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;  // 0 stage only, 1 unmasked, 2 masked
    const int buf = kt & 1;
    if (kt + 1 < n_kt) prefetch((kt + 1) * kBK);
    if constexpr (MODE == 1) tile_step(buf, kt * kBK, std::false_type{});
    if constexpr (MODE == 2) tile_step(buf, kt * kBK, std::true_type{});
    if (kt + 1 < n_kt) stage(buf ^ 1);
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 1 < n_kt_w; ++kt) iteration(kt, std::integral_constant<int, 1>{});
  if (kt < n_kt_w) {
    iteration(kt, std::integral_constant<int, 2>{});
    ++kt;
  }
  for (; kt < n_kt; ++kt) iteration(kt, std::integral_constant<int, 0>{});

  if (!wave_active) return;
  const float l_tot = pair_sum(l_run);
  if (my_q < n) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = out + (int64_t)(lo + my_q) * ((int64_t)Hq * HD) + (int64_t)h * HD;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * G;
        unsigned w[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const __bf16 e0 = (__bf16)(o[db][4 * g4 + 2 * j] * inv);
          const __bf16 e1 = (__bf16)(o[db][4 * g4 + 2 * j + 1] * inv);
          w[j] = (unsigned)__builtin_bit_cast(uint16_t, e0) |
                 ((unsigned)__builtin_bit_cast(uint16_t, e1) << 16);
        }
        *reinterpret_cast<uint2*>(op + d0) = make_uint2(w[0], w[1]);
      }
    if (lse != nullptr && G == 0) lse[(int64_t)h * Kt + lo + my_q] = (m_run * qk_scale + __log2f(l_tot)) * kLn2;
  }
}

template <int HD>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    int64_t qs, int64_t ks, int64_t vs, const float* __restrict__ bias,
    const float* __restrict__ gain, float qk_scale, const int32_t* __restrict__ cu, int Hq,
    int group, int64_t Kt, float* __restrict__ out, float* __restrict__ lse) {
  const int b = blockIdx.y, h = blockIdx.z;
  const int lo = cu[b], n = cu[b + 1] - lo;
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= n) return;
  const int kvh = h / group;
  const float gmul = gain ? gain[h] * kLog2e : 0.0f;
  float qr[HD], acc[HD];
  const float* qp = q + (int64_t)(lo + i) * qs + (int64_t)h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qr[d] = qp[d];
    acc[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int j = 0; j <= i; ++j) {
    const float* kp = k + (int64_t)(lo + j) * ks + (int64_t)kvh * HD;
    const float* vp = v + (int64_t)(lo + j) * vs + (int64_t)kvh * HD;
    float dot = 0.0f;
#pragma unroll
    for (int d = 0; d < HD; ++d) dot = fmaf(qr[d], kp[d], dot);
    const float y = dot * qk_scale + (bias ? gmul * bias[lo + j] : 0.0f);
    const float m_new = fmaxf(m, y);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(y - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int d = 0; d < HD; ++d) acc[d] = fmaf(p, vp[d], acc[d] * alpha);
    m = m_new;
  }
  float* op = out + (int64_t)(lo + i) * ((int64_t)Hq * HD) + (int64_t)h * HD;
#pragma unroll
  for (int d = 0; d < HD; ++d) op[d] = acc[d] / l;
  if (lse != nullptr) lse[(int64_t)h * Kt + lo + i] = (m + log2f(l)) * kLn2;
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, int64_t qs, int64_t ks,
                            int64_t vs, const float* bias, const float* gain, float tau,
                            const int32_t* cu_kept, int B, int max_len, int64_t Kt, int Hq,
                            int Hkv, int d, void* out, float* lse, hipStream_t s) {
  if (B == 0 || max_len == 0) return hipSuccess;
  const int group = Hq / Hkv;
  // head_dim 128: TG_ATTN_WAVES waves (32 query rows each) per workgroup;
  // head_dim 64: 4 waves (a 64x64 V tile gives 256 transpose items).
  constexpr int NW = TG_ATTN_WAVES;
  const int swz = (Hq % 8 == 0 && ((Hq / 8) % group) == 0) ? 1 : 0;
  const float qk_scale = tau * kLog2e / sqrtf((float)d);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(out);
  if (d == 128) {
    const int n_qtiles = (max_len + 32 * NW - 1) / (32 * NW);
    const dim3 grid((unsigned)Hq, (unsigned)B, (unsigned)n_qtiles);
    hipLaunchKernelGGL((attn_bf16_kernel<128, NW>), grid, dim3(64 * NW), 0, s, qq, kk, vv, qs, ks,
                       vs, bias, gain, qk_scale, cu_kept, Hq, group, swz, n_qtiles, Kt, oo, lse);
  } else if (d == 64) {
    const int n_qtiles = (max_len + 127) / 128;
    const dim3 grid((unsigned)Hq, (unsigned)B, (unsigned)n_qtiles);
    hipLaunchKernelGGL((attn_bf16_kernel<64, 4>), grid, dim3(256), 0, s, qq, kk, vv, qs, ks, vs,
                       bias, gain, qk_scale, cu_kept, Hq, group, swz, n_qtiles, Kt, oo, lse);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, int64_t qs, int64_t ks,
                           int64_t vs, const float* bias, const float* gain, float tau,
                           const int32_t* cu_kept, int B, int max_len, int64_t Kt, int Hq,
                           int Hkv, int d, float* out, float* lse, hipStream_t s) {
  if (B == 0 || max_len == 0) return hipSuccess;
  const int group = Hq / Hkv;
  const float qk_scale = tau * kLog2e / sqrtf((float)d);
  const dim3 grid((unsigned)((max_len + 63) / 64), (unsigned)B, (unsigned)Hq);
  if (d == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, s, q, k, v, qs, ks, vs, bias, gain,
                       qk_scale, cu_kept, Hq, group, Kt, out, lse);
  else if (d == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, s, q, k, v, qs, ks, vs, bias, gain,
                       qk_scale, cu_kept, Hq, group, Kt, out, lse);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tg

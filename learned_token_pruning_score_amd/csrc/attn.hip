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
//    16-key MFMA step, lane half G holds keys 4G..4G+3 and 8+4G..8+4G+3), so
//    V is staged transposed in LDS and read as two 8-byte runs.
//  * K rows and V^T rows are XOR-swizzled in LDS so fragment reads of 32
//    rows spread over all banks.
//  * Causal masking only on tiles that cross the wave's diagonal; tiles are
//    launched longest-first (tile index is the slowest grid dimension,
//    reversed); the heads of one GQA group land on the same XCD.
// fp32 path: one thread per (row, head), online softmax on vector ALUs.
#include <math.h>

#include "tg_common.h"

namespace tg {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBQ = 128;  // query rows per workgroup
constexpr int kBK = 64;   // keys per tile

template <int HD>
__device__ __forceinline__ int kswz(int r, int c) {
  // K rows are HD*2 bytes: 256 B (HD=128) or 128 B (HD=64).
  return HD == 128 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}
// V^T rows are 64 keys * 2 B = 128 B = 16 units of 8 B.
__device__ __forceinline__ int vswz(int d, int u) { return u ^ ((d >> 1) & 15); }

__device__ __forceinline__ unsigned elem16(const uint4& v, int e) {
  const unsigned w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int HD>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t qs, int64_t ks, int64_t vs,
    const float* __restrict__ bias, const float* __restrict__ gain, float qk_scale,
    const int32_t* __restrict__ cu, int Hq, int group, int head_swizzle, int n_qtiles,
    int64_t Kt, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int KCH = HD / 8;   // 16-byte chunks per K row
  constexpr int NKS = HD / 16;  // MFMA k-steps over the head dim
  constexpr int NDB = HD / 32;  // 32-row blocks of O^T
  __shared__ uint4 sK[kBK * KCH];
  __shared__ uint2 sVt[HD * (kBK / 4)];
  __shared__ float sB[kBK];

  const int x = blockIdx.x;
  const int h = head_swizzle ? (x % 8) * (Hq / 8) + x / 8 : x;
  const int b = blockIdx.y;
  const int tile = n_qtiles - 1 - (int)blockIdx.z;
  const int lo = cu[b];
  const int n = cu[b + 1] - lo;
  const int q0 = tile * kBQ;
  if (q0 >= n) return;
  const int kvh = h / group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = lane >> 5;
  const int qw = q0 + wave * 32;
  const int my_q = qw + (lane & 31);
  const float gmul = gain ? gain[h] * kLog2e : 0.0f;

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
  float m_run = -INFINITY, l_run = 0.0f;

  const int kv_end = min(q0 + kBQ, n);
  const int n_kt = (kv_end + kBK - 1) / kBK;
  const bool wave_active = qw < n;
  const int n_kt_w = wave_active ? min(qw + 31, n - 1) / kBK + 1 : 0;
  const uint16_t* kbase = k + (int64_t)lo * ks + (int64_t)kvh * HD;
  const uint16_t* vbase = v + (int64_t)lo * vs + (int64_t)kvh * HD;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * kBK;
    __syncthreads();
    for (int id = tid; id < kBK * KCH; id += 256) {
      const int r = id / KCH, c = id % KCH;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (k0 + r < n) val = *reinterpret_cast<const uint4*>(kbase + (int64_t)(k0 + r) * ks + c * 8);
      sK[r * KCH + kswz<HD>(r, c)] = val;
    }
    for (int id = tid; id < 16 * KCH; id += 256) {
      const int kg = id % 16, dc = id / 16;
      uint4 rows[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 4 * kg + j;
        rows[j] = make_uint4(0, 0, 0, 0);
        if (key < n) rows[j] = *reinterpret_cast<const uint4*>(vbase + (int64_t)key * vs + dc * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = dc * 8 + e;
        uint2 u;
        u.x = elem16(rows[0], e) | (elem16(rows[1], e) << 16);
        u.y = elem16(rows[2], e) | (elem16(rows[3], e) << 16);
        sVt[d * 16 + vswz(d, kg)] = u;
      }
    }
    if (tid < kBK) sB[tid] = (bias != nullptr && k0 + tid < n) ? bias[lo + k0 + tid] * gmul : 0.0f;
    __syncthreads();
    if (kt >= n_kt_w) continue;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
      const int r = kb * 32 + (lane & 31);
#pragma unroll
      for (int st = 0; st < NKS; ++st)
        s[kb] = mfma32x32x16(as_bf16x8(sK[r * KCH + kswz<HD>(r, 2 * st + G)]), qf[st], s[kb]);
    }

    const bool diag = (k0 + kBK - 1) > qw;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + acc_row(i, lane);
        float y = fmaf(s[kb][i], qk_scale, sB[key]);
        if (diag && (k0 + key) > my_q) y = -INFINITY;
        s[kb][i] = y;
        mx = fmaxf(mx, y);
      }
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[kb][i] - m_new);
        s[kb][i] = p;
        psum += p;
      }
    l_run = fmaf(l_run, alpha, psum);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }
    m_run = m_new;

    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[kb][hh][j] = (__bf16)s[kb][8 * hh + j];

#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + (lane & 31);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int u0 = kb * 8 + 4 * hh + G;
          const uint2 a0 = sVt[d * 16 + vswz(d, u0)];
          const uint2 a1 = sVt[d * 16 + vswz(d, u0 + 2)];
          const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
          o[db] = mfma32x32x16(as_bf16x8(a), pb[kb][hh], o[db]);
        }
    }
  }

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
    if (lse != nullptr && G == 0) lse[(int64_t)h * Kt + lo + my_q] = (m_run + __log2f(l_tot)) * kLn2;
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
  const int n_qtiles = (max_len + kBQ - 1) / kBQ;
  const int swz = (Hq % 8 == 0 && ((Hq / 8) % group) == 0) ? 1 : 0;
  const float qk_scale = tau * kLog2e / sqrtf((float)d);
  const dim3 grid((unsigned)Hq, (unsigned)B, (unsigned)n_qtiles);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(out);
  if (d == 128)
    hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, s, qq, kk, vv, qs, ks, vs, bias,
                       gain, qk_scale, cu_kept, Hq, group, swz, n_qtiles, Kt, oo, lse);
  else if (d == 64)
    hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, s, qq, kk, vv, qs, ks, vs, bias,
                       gain, qk_scale, cu_kept, Hq, group, swz, n_qtiles, Kt, oo, lse);
  else
    return hipErrorInvalidValue;
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

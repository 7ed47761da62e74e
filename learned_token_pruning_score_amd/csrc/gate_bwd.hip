// Backward of the gate MLP (TokenGate article, section "What is
// token-gated attention?": the kept token's score enters the attention
// above the gate as a logit bias, which is the scorer's gradient path; top-K
// itself passes no gradient).  The score of token t is
//     s_t = b2 + w2 . silu(a_t),  a_t = W1 h_t + b1
// and a kept document token's bias is its score, so ds_t is the bias
// gradient of its kept row (summed over the pruned layers by the caller);
// every other token gets none.  Then
//     dw2 = sum_t ds_t silu(a_t)    db2 = sum_t ds_t
//     da_t = ds_t w2 * silu'(a_t)   db1 = sum_t da_t
//     dW1 = sum_t da_t h_t^T        dh_t = W1^T da_t
// over the kept rows only (ds is zero elsewhere).  bf16 path:
//   gbwd_ds       ds of each kept row (its bias gradient inside the
//                 document, 0 outside), from kept_idx and the spans.
//   gbwd_a        a = W1 h recomputed split over K (fp32 partials per chunk
//                 of columns; at the kept rows' height a 256-row tile per CU
//                 would leave most of the chip idle).
//   gbwd_da_finish  a = sum of the chunks + b1, da (bf16) and fixed-order
//                 per-32-row column sums of da and ds silu(a).
//   dh            the projection kernel on da with W1 transposed.
//   gbwd_dw1      dW1 = da^T h: one workgroup per (64-column slice of h, chunk
//                 of rows), both MFMA operands through transposing LDS reads
//                 of the row-major tiles, fp32 partial sums per chunk.
//   sums          dW1, db1, dw2, db2 as fixed-order sums of the partials.
// fp32 path: one thread per output element on vector ALUs.
#include <math.h>

#include "tg_common.h"

namespace tg {
namespace {

constexpr int kBufFlagsG = 0x00020000;  // raw buffer: reads past num_records give 0
constexpr int kGR = 64;                 // rows per stage of gbwd_dw1

typedef short gs4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) gs4 lds_gs4;
typedef unsigned gu4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const gu4 g_lds_u4;

__device__ __forceinline__ uint32_t g_lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(reinterpret_cast<const char*>(p));
}

// Transposed 32-column fragment of a row-major LDS tile (rows of RU 16-byte
// units): lane l receives rows 4G..4G+3 and 8+4G..8+4G+3 (G = l / 32) of the
// 16-row step kh, column l % 32 of block cb.  Used for both operands, so the
// MFMA's k index runs over the same 16 rows in the same order on both sides.
template <int RU>
__device__ __forceinline__ bf16x8 g_frag_tr(uint32_t tbase, int kh, int cb) {
  const uint32_t a0 = tbase + (16 * kh) * (RU * 16) + cb * 64;
  const gs4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_gs4*)(uintptr_t)a0);
  const gs4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_gs4*)(uintptr_t)(a0 + 8 * (RU * 16)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int RU>
__device__ __forceinline__ uint32_t g_tr_base(const void* tile, int lane) {
  const int gi = lane & 15, g = lane >> 4;
  return g_lds_addr(reinterpret_cast<const char*>(tile) + (4 * (g >> 1) + (gi >> 2)) * (RU * 16) +
                    (16 * (g & 1) + 4 * (gi & 3)) * 2);
}

// Pre-activation a = W1 h (without b1) of the kept rows, split over K:
// workgroup (128-row tile, K chunk) writes its fp32 partial
// part[chunk][row][f] for all F columns.  Both operands are K-contiguous
// (rows of h and of W1), so MFMA fragments are plain 16-byte row reads:
// lane l supplies row l % 32, columns 8 (l / 32) .. +7 of a 16-column step,
// for W1 (A operand, rows f) and for h (B operand, rows = tokens); register
// i of lane l then holds a[token l % 32][f = acc_row(i, l)].  Wave w owns the
// 32-column blocks w, w + 4 of f and all 128 rows; a 64-column stage of
// W1 (F rows) and h (128 rows) sits in LDS with rows padded to 9 16-byte
// units (conflict-free reads), the next stage's loads in registers.
template <int F>
__global__ __launch_bounds__(256, 2) void gbwd_a_kernel(const uint16_t* __restrict__ h, int64_t ld, int64_t Kt, int D,
                                                        const uint16_t* __restrict__ W1, int kc_cols,
                                                        float* __restrict__ part) {
  constexpr int RU = 9;
  constexpr int NFB = F / 32;
  constexpr int FBW = (NFB + 3) / 4;       // f-blocks per wave
  constexpr int W_ITEMS = F * 8 / 256;     // 16-byte chunks per thread of a W1 stage
  constexpr int H_ITEMS = 128 * 8 / 256;
  __shared__ uint4 sW[F * RU], sH[128 * RU];
  const int64_t t0 = (int64_t)blockIdx.x * 128;
  const int chunk = blockIdx.y;
  const int k_begin = chunk * kc_cols;
  const int k_end = min(D, k_begin + kc_cols);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 5;
  const int rows = __builtin_amdgcn_readfirstlane((int)min((int64_t)128, Kt - t0));
  f32x16 acc[FBW][4];
#pragma unroll
  for (int a = 0; a < FBW; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  uint4 vw[W_ITEMS], vh[H_ITEMS];
  auto prefetch = [&](int k0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W1 + k0), (short)0, (F - 1) * D * 2 + 128, kBufFlagsG);
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc((void*)(h + t0 * ld + k0), (short)0, rows * (int)ld * 2, kBufFlagsG);
#pragma unroll
    for (int j = 0; j < W_ITEMS; ++j) {
      const int id = tid + 256 * j;
      vw[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, ((id / 8) * D + (id % 8) * 8) * 2, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < H_ITEMS; ++j) {
      const int id = tid + 256 * j;
      vh[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, ((id / 8) * (int)ld + (id % 8) * 8) * 2, 0, 0));
    }
  };
  uint32_t wl = g_lds_addr(sW) + ((lane & 31) * RU + G) * 16, hl = g_lds_addr(sH) + ((lane & 31) * RU + G) * 16;
  asm volatile("" : "+v"(wl), "+v"(hl));
  prefetch(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += 64) {
    __syncthreads();  // the previous stage is no longer read
#pragma unroll
    for (int j = 0; j < W_ITEMS; ++j) {
      const int id = tid + 256 * j;
      sW[(id / 8) * RU + id % 8] = vw[j];
    }
#pragma unroll
    for (int j = 0; j < H_ITEMS; ++j) {
      const int id = tid + 256 * j;
      sH[(id / 8) * RU + id % 8] = vh[j];
    }
    __syncthreads();
    if (k0 + 64 < k_end) prefetch(k0 + 64);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8 hf[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        hf[b] = __builtin_bit_cast(bf16x8, *(g_lds_u4*)(uintptr_t)(hl + ((32 * b) * RU + 2 * st) * 16));
#pragma unroll
      for (int a = 0; a < FBW; ++a) {
        const int fb = wave + 4 * a;
        if (fb < NFB) {
          const bf16x8 wf = __builtin_bit_cast(bf16x8, *(g_lds_u4*)(uintptr_t)(wl + ((32 * fb) * RU + 2 * st) * 16));
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = mfma32x32x16(wf, hf[b], acc[a][b]);
        }
      }
    }
  }
  // acc[a][b]: f = 32 (wave + 4a) + acc_row(i, lane), row t0 + 32 b + lane % 32
  float* pc = part + (int64_t)chunk * Kt * F;
#pragma unroll
  for (int a = 0; a < FBW; ++a) {
    const int fb = wave + 4 * a;
    if (fb < NFB) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t t = t0 + 32 * b + (lane & 31);
        if (t < Kt) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<float4*>(pc + t * F + 32 * fb + 8 * g4 + 4 * G) =
                make_float4(acc[a][b][4 * g4], acc[a][b][4 * g4 + 1], acc[a][b][4 * g4 + 2], acc[a][b][4 * g4 + 3]);
        }
      }
    }
  }
}

// da from the partials: workgroup (32-row block, 64 columns), thread
// (quarter q, column f) takes rows 8q .. 8q + 7 of the block: a = (sum of the
// chunks in order) + b1, da = ds w2 silu'(a) (bf16), and the column sums of
// da and ds silu(a) over its rows in order, then over the quarters in order.
__global__ __launch_bounds__(256) void gbwd_da_finish_kernel(const float* __restrict__ part, int n_kc, int64_t Kt,
                                                             int F, const float* __restrict__ b1,
                                                             const float* __restrict__ w2, const float* __restrict__ ds,
                                                             uint16_t* __restrict__ da, float* __restrict__ p1,
                                                             float* __restrict__ p2) {
  __shared__ float r1[4][64], r2[4][64];
  const int tid = threadIdx.x;
  const int q = tid >> 6, c = tid & 63;
  const int f = blockIdx.y * 64 + c;
  const int64_t blk = blockIdx.x;
  float c1 = 0.0f, c2 = 0.0f;
  if (f < F) {
    const float bb = b1 ? b1[f] : 0.0f, ww = w2[f];
    const int64_t r0 = blk * 32 + 8 * q;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t t = r0 + j;
      if (t < Kt) {
        float a = part[t * F + f];
        for (int k = 1; k < n_kc; ++k) a += part[((int64_t)k * Kt + t) * F + f];
        a += bb;
        const float dsr = ds[t];
        const float sg = 1.0f / (1.0f + expf(-a));
        const float d = dsr * ww * sg * (1.0f + a * (1.0f - sg));
        da[t * F + f] = __builtin_bit_cast(uint16_t, (__bf16)d);
        c1 += d;
        c2 += dsr * a * sg;
      }
    }
  }
  r1[q][c] = c1;
  r2[q][c] = c2;
  __syncthreads();
  if (q == 0 && f < F) {
    p1[blk * F + f] = ((r1[0][c] + r1[1][c]) + r1[2][c]) + r1[3][c];
    p2[blk * F + f] = ((r2[0][c] + r2[1][c]) + r2[2][c]) + r2[3][c];
  }
}

__global__ __launch_bounds__(256) void gbwd_fill_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// ds of each kept row: its bias gradient when the row's token lies inside
// its prompt's document, else 0.
__global__ __launch_bounds__(256) void gbwd_ds_kernel(const float* __restrict__ dbias, const int32_t* __restrict__ kept_idx,
                                                      const int32_t* __restrict__ cu, const int32_t* __restrict__ db,
                                                      const int32_t* __restrict__ de, int B, int64_t Kt,
                                                      float* __restrict__ ds) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= Kt) return;
  const int t = kept_idx[r];
  int lo = 0, hi = B;  // prompt b with cu[b] <= t < cu[b + 1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int rel = t - cu[lo];
  ds[r] = (rel >= db[lo] && rel < de[lo]) ? dbias[r] : 0.0f;
}

// W1 [F, D] -> W1^T [D, F], one thread per element.
__global__ __launch_bounds__(256) void gbwd_transpose_kernel(const uint16_t* __restrict__ w, int F, int D,
                                                             uint16_t* __restrict__ wt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)F * D) return;
  const int64_t dcol = i / F;
  const int f = (int)(i - dcol * F);
  wt[i] = w[(int64_t)f * D + dcol];
}

// dW1 partial of one chunk of rows: C[f][d] = sum_t da[t][f] h[t][d] for the
// 64 columns [d0, d0 + 64) of h.  4 waves; wave w owns the 32-row blocks
// {w, w + 4} of F and both 32-column blocks of the slice.
template <int F>
__global__ __launch_bounds__(256) void gbwd_dw1_kernel(const uint16_t* __restrict__ da, const uint16_t* __restrict__ h,
                                                       int64_t ld, int64_t Kt, int D, int chunk_rows,
                                                       float* __restrict__ part) {
  constexpr int RA = F / 8 + 4;   // 16-byte units per padded da row
  constexpr int RH = 64 / 8 + 4;  // 16-byte units per padded h row (64 columns)
  constexpr int NFB = F / 32;
  constexpr int A_ITEMS = kGR * (F / 8) / 256;
  constexpr int H_ITEMS = kGR * 8 / 256;
  __shared__ uint4 sA[kGR * RA], sH[kGR * RH];
  const int d0 = blockIdx.x * 64;
  const int chunk = blockIdx.y;
  const int64_t r0 = (int64_t)chunk * chunk_rows;
  const int64_t r_end = min(r0 + chunk_rows, Kt);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
  const uint32_t abase = g_tr_base<RA>(sA, lane), hbase = g_tr_base<RH>(sH, lane);
  for (int64_t rs = r0; rs < r_end; rs += kGR) {
    const int rows = __builtin_amdgcn_readfirstlane((int)min((int64_t)kGR, r_end - rs));
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)(da + rs * F), (short)0, rows * F * 2, kBufFlagsG);
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc((void*)(h + rs * ld + d0), (short)0, rows * (int)ld * 2, kBufFlagsG);
    uint4 va[A_ITEMS], vh[H_ITEMS];
#pragma unroll
    for (int j = 0; j < A_ITEMS; ++j) {
      const int id = tid + 256 * j;
      va[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra, ((id / (F / 8)) * F + (id % (F / 8)) * 8) * 2, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < H_ITEMS; ++j) {
      const int id = tid + 256 * j;
      vh[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, ((id / 8) * (int)ld + (id % 8) * 8) * 2, 0, 0));
    }
    __syncthreads();  // the previous stage is no longer read
#pragma unroll
    for (int j = 0; j < A_ITEMS; ++j) {
      const int id = tid + 256 * j;
      sA[(id / (F / 8)) * RA + id % (F / 8)] = va[j];
    }
#pragma unroll
    for (int j = 0; j < H_ITEMS; ++j) {
      const int id = tid + 256 * j;
      sH[(id / 8) * RH + id % 8] = vh[j];
    }
    __syncthreads();
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) {
      const bf16x8 b0 = g_frag_tr<RH>(hbase, kh, 0), b1 = g_frag_tr<RH>(hbase, kh, 1);
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int fb = wave + 4 * a;
        if (fb < NFB) {
          const bf16x8 af = g_frag_tr<RA>(abase, kh, fb);
          acc[a][0] = mfma32x32x16(af, b0, acc[a][0]);
          acc[a][1] = mfma32x32x16(af, b1, acc[a][1]);
        }
      }
    }
  }
  // acc[a][b]: rows f = 32 (wave + 4a) + acc_row(i, lane), column d0 + 32 b + lane % 32
  float* pc = part + (int64_t)chunk * F * D;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int fb = wave + 4 * a;
    if (fb < NFB) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          pc[(int64_t)(32 * fb + acc_row(i, lane)) * D + d0 + 32 * b + (lane & 31)] = acc[a][b][i];
    }
  }
}

// Fixed-order sums of the partials.  dW1: one thread per element over the
// chunks.  db1 / dw2: one workgroup per 64 columns; thread (g, c) sums the
// 32-row blocks g, g + 4, ... of column c, then the four partials are added
// in order.  db2: one workgroup, a strided sum per thread, then a tree.
__global__ __launch_bounds__(256) void gbwd_dw1_sum_kernel(const float* __restrict__ part, int n_chunks, int64_t FD,
                                                           float* __restrict__ dW1) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= FD) return;
  float acc = 0.0f;
  for (int c = 0; c < n_chunks; ++c) acc += part[(int64_t)c * FD + i];
  dW1[i] = acc;
}

// db1 and dw2 from the per-32-row-block column sums: 64 columns per
// workgroup, 16 groups of blocks (block b in group b % 16) per column, the
// group sums added in group order.
__global__ __launch_bounds__(1024) void gbwd_col_sum_kernel(const float* __restrict__ p1, const float* __restrict__ p2,
                                                            int64_t n_blk, int F, float* __restrict__ db1,
                                                            float* __restrict__ dw2) {
  constexpr int NG = 16;
  __shared__ float r1[NG][64], r2[NG][64];
  const int tid = threadIdx.x;
  const int grp = tid >> 6;
  const int f = blockIdx.x * 64 + (tid & 63);
  float a1 = 0.0f, a2 = 0.0f;
  if (f < F) {
#pragma unroll 8
    for (int64_t b = grp; b < n_blk; b += NG) {
      a1 += p1[b * F + f];
      a2 += p2[b * F + f];
    }
  }
  r1[grp][tid & 63] = a1;
  r2[grp][tid & 63] = a2;
  __syncthreads();
  if (tid < 64 && f < F) {
    float s1 = r1[0][tid], s2 = r2[0][tid];
#pragma unroll
    for (int g = 1; g < NG; ++g) {
      s1 += r1[g][tid];
      s2 += r2[g][tid];
    }
    if (db1) db1[f] = s1;
    dw2[f] = s2;
  }
}

// db2 = sum of ds: thread i sums rows i, i + 1024, ... (loads unrolled), then
// a fixed tree over the 1024 threads.
__global__ __launch_bounds__(1024) void gbwd_sum_ds_kernel(const float* __restrict__ ds, int64_t Kt, float* __restrict__ db2) {
  __shared__ float red[1024];
  const int tid = threadIdx.x;
  float acc = 0.0f;
#pragma unroll 8
  for (int64_t r = tid; r < Kt; r += 1024) acc += ds[r];
  red[tid] = acc;
  __syncthreads();
  for (int w = 512; w >= 1; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) *db2 = red[0];
}

// ---------------------------------------------------------------- fp32
__global__ __launch_bounds__(256) void gbwd_da_f32_kernel(const float* __restrict__ h, int64_t ld, int64_t Kt, int D,
                                                          const float* __restrict__ W1, const float* __restrict__ b1,
                                                          const float* __restrict__ w2, int F, const float* __restrict__ ds,
                                                          float* __restrict__ da, float* __restrict__ zds) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Kt * F) return;
  const int64_t r = i / F;
  const int f = (int)(i - r * F);
  float a = b1 ? b1[f] : 0.0f;
  for (int k = 0; k < D; ++k) a = fmaf(W1[(int64_t)f * D + k], h[r * ld + k], a);
  const float sg = 1.0f / (1.0f + expf(-a));
  da[i] = ds[r] * w2[f] * sg * (1.0f + a * (1.0f - sg));
  zds[i] = ds[r] * a * sg;
}

__global__ __launch_bounds__(256) void gbwd_dh_f32_kernel(const float* __restrict__ da, int64_t Kt, int F,
                                                          const float* __restrict__ W1, int D, float* __restrict__ dh) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Kt * D) return;
  const int64_t r = i / D;
  const int d = (int)(i - r * D);
  float a = 0.0f;
  for (int f = 0; f < F; ++f) a = fmaf(da[r * F + f], W1[(int64_t)f * D + d], a);
  dh[i] = a;
}

__global__ __launch_bounds__(256) void gbwd_dw1_f32_kernel(const float* __restrict__ da, const float* __restrict__ h,
                                                           int64_t ld, int64_t Kt, int F, int D, const float* __restrict__ zds,
                                                           const float* __restrict__ ds, float* __restrict__ dW1,
                                                           float* __restrict__ db1, float* __restrict__ dw2,
                                                           float* __restrict__ db2) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t FD = (int64_t)F * D;
  if (i < FD) {
    const int f = (int)(i / D);
    const int d = (int)(i - (int64_t)f * D);
    float a = 0.0f;
    for (int64_t r = 0; r < Kt; ++r) a = fmaf(da[r * F + f], h[r * ld + d], a);
    dW1[i] = a;
  } else if (i < FD + F) {
    const int f = (int)(i - FD);
    float a1 = 0.0f, a2 = 0.0f;
    for (int64_t r = 0; r < Kt; ++r) {
      a1 += da[r * F + f];
      a2 += zds[r * F + f];
    }
    if (db1) db1[f] = a1;
    dw2[f] = a2;
  } else if (i == FD + F) {
    float acc = 0.0f;
    for (int64_t r = 0; r < Kt; ++r) acc += ds[r];
    *db2 = acc;
  }
}

size_t galign(size_t x) { return (x + 255) & ~(size_t)255; }

struct GbwdLayout {
  int64_t n_blk;       // 32-row blocks of the da column sums
  int chunk_rows;      // rows per dW1 chunk
  int n_chunks;
  int kc_cols;         // columns of h per K chunk of the pre-activation
  int n_kc;
  size_t off_ds, off_da, off_wt, off_p1, off_p2, off_part, off_pa, total;
};

GbwdLayout gbwd_layout(int64_t Kt, int D, int F, int eb) {
  GbwdLayout L{};
  L.n_blk = (Kt + 31) / 32;
  // K chunks of the pre-activation: enough (128-row tile, chunk) workgroups
  // for every CU, in whole 64-column stages
  const int64_t a_tiles = (Kt + 127) / 128;
  const int64_t n_stage = D / 64;
  int64_t kc = a_tiles > 0 ? (256 + a_tiles - 1) / a_tiles : 1;
  if (kc > n_stage) kc = n_stage;
  if (kc < 1) kc = 1;
  L.kc_cols = (int)((n_stage + kc - 1) / kc * 64);
  L.n_kc = (int)((D + L.kc_cols - 1) / L.kc_cols);
  const int64_t row_tiles = (Kt + kGR - 1) / kGR;
  const int n_dt = D / 64;
  int64_t want = (256 + n_dt - 1) / n_dt;
  if (want < 1) want = 1;
  if (want > row_tiles) want = row_tiles > 0 ? row_tiles : 1;
  L.chunk_rows = (int)(((row_tiles + want - 1) / want) * kGR);
  if (L.chunk_rows < kGR) L.chunk_rows = kGR;  // no rows: one empty chunk
  L.n_chunks = (int)((Kt + L.chunk_rows - 1) / L.chunk_rows);
  if (L.n_chunks < 1) L.n_chunks = 1;
  size_t o = 0;
  L.off_ds = o; o += galign((size_t)Kt * 4);
  L.off_da = o; o += galign((size_t)Kt * F * eb);
  if (eb == 2) {
    L.off_wt = o; o += galign((size_t)D * F * 2);
    L.off_p1 = o; o += galign((size_t)L.n_blk * F * 4);
    L.off_p2 = o; o += galign((size_t)L.n_blk * F * 4);
    L.off_part = o; o += galign((size_t)L.n_chunks * F * D * 4);
    L.off_pa = o; o += galign((size_t)L.n_kc * Kt * F * 4);
  } else {
    L.off_p2 = o; o += galign((size_t)Kt * F * 4);  // ds * silu(a) per element
  }
  L.total = o;
  return L;
}

}  // namespace

size_t gate_bwd_workspace_bytes(int64_t Kt, int D, int F, int elem_bytes) {
  return gbwd_layout(Kt, D, F, elem_bytes).total;
}

hipError_t launch_gate_bwd(const void* h, int64_t ld, int64_t Kt, int D, const void* W1, const float* b1,
                           const float* w2, int F, const float* dbias, const int32_t* kept_idx,
                           const int32_t* cu, const int32_t* db, const int32_t* de, int B, int elem_bytes,
                           void* dh, float* dW1, float* db1, float* dw2, float* db2, void* ws,
                           hipStream_t s) {
  const dim3 blk(256);
  if (Kt == 0) {  // no kept rows: every gradient is zero
    const int64_t FD = (int64_t)F * D;
    hipLaunchKernelGGL(gbwd_fill_kernel, dim3((unsigned)((FD + 255) / 256)), blk, 0, s, dW1, FD);
    if (db1) hipLaunchKernelGGL(gbwd_fill_kernel, dim3((unsigned)((F + 255) / 256)), blk, 0, s, db1, (int64_t)F);
    hipLaunchKernelGGL(gbwd_fill_kernel, dim3((unsigned)((F + 255) / 256)), blk, 0, s, dw2, (int64_t)F);
    hipLaunchKernelGGL(gbwd_fill_kernel, dim3(1), blk, 0, s, db2, (int64_t)1);
    return hipGetLastError();
  }
  const GbwdLayout L = gbwd_layout(Kt, D, F, elem_bytes);
  char* w = static_cast<char*>(ws);
  float* ds = reinterpret_cast<float*>(w + L.off_ds);
  hipLaunchKernelGGL(gbwd_ds_kernel, dim3((unsigned)((Kt + 255) / 256)), blk, 0, s, dbias, kept_idx, cu, db, de, B,
                     Kt, ds);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_red = (int64_t)F * D + F + 1;
  if (elem_bytes == 2) {
    void* da = w + L.off_da;
    uint16_t* wt = reinterpret_cast<uint16_t*>(w + L.off_wt);
    float* p1 = reinterpret_cast<float*>(w + L.off_p1);
    float* p2 = reinterpret_cast<float*>(w + L.off_p2);
    float* part = reinterpret_cast<float*>(w + L.off_part);
    float* pa = reinterpret_cast<float*>(w + L.off_pa);
    const auto* hp = static_cast<const uint16_t*>(h);
    const auto* w1p = static_cast<const uint16_t*>(W1);
    const dim3 ga((unsigned)((Kt + 127) / 128), (unsigned)L.n_kc);
    if (F == 256) hipLaunchKernelGGL(gbwd_a_kernel<256>, ga, blk, 0, s, hp, ld, Kt, D, w1p, L.kc_cols, pa);
    else if (F == 128) hipLaunchKernelGGL(gbwd_a_kernel<128>, ga, blk, 0, s, hp, ld, Kt, D, w1p, L.kc_cols, pa);
    else hipLaunchKernelGGL(gbwd_a_kernel<64>, ga, blk, 0, s, hp, ld, Kt, D, w1p, L.kc_cols, pa);
    hipLaunchKernelGGL(gbwd_da_finish_kernel, dim3((unsigned)L.n_blk, (unsigned)((F + 63) / 64)), blk, 0, s, pa, L.n_kc,
                       Kt, F, b1, w2, ds, static_cast<uint16_t*>(da), p1, p2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gbwd_transpose_kernel, dim3((unsigned)(((int64_t)F * D + 255) / 256)), blk, 0, s,
                       static_cast<const uint16_t*>(W1), F, D, wt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_proj_store(da, F, Kt, F, wt, D, dh, D, s);
    if (e != hipSuccess) return e;
    const dim3 g((unsigned)(D / 64), (unsigned)L.n_chunks);
    const auto* dap = static_cast<const uint16_t*>(da);
    if (F == 256) hipLaunchKernelGGL(gbwd_dw1_kernel<256>, g, blk, 0, s, dap, hp, ld, Kt, D, L.chunk_rows, part);
    else if (F == 128) hipLaunchKernelGGL(gbwd_dw1_kernel<128>, g, blk, 0, s, dap, hp, ld, Kt, D, L.chunk_rows, part);
    else hipLaunchKernelGGL(gbwd_dw1_kernel<64>, g, blk, 0, s, dap, hp, ld, Kt, D, L.chunk_rows, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t FD = (int64_t)F * D;
    hipLaunchKernelGGL(gbwd_dw1_sum_kernel, dim3((unsigned)((FD + 255) / 256)), blk, 0, s, part, L.n_chunks, FD, dW1);
    hipLaunchKernelGGL(gbwd_col_sum_kernel, dim3((unsigned)((F + 63) / 64)), dim3(1024), 0, s, p1, p2, L.n_blk, F,
                       db1, dw2);
    hipLaunchKernelGGL(gbwd_sum_ds_kernel, dim3(1), dim3(1024), 0, s, ds, Kt, db2);
    return hipGetLastError();
  }
  float* da = reinterpret_cast<float*>(w + L.off_da);
  float* zds = reinterpret_cast<float*>(w + L.off_p2);
  const auto* hp = static_cast<const float*>(h);
  const auto* wp = static_cast<const float*>(W1);
  hipLaunchKernelGGL(gbwd_da_f32_kernel, dim3((unsigned)((Kt * F + 255) / 256)), blk, 0, s, hp, ld, Kt, D, wp, b1, w2,
                     F, ds, da, zds);
  hipLaunchKernelGGL(gbwd_dh_f32_kernel, dim3((unsigned)((Kt * D + 255) / 256)), blk, 0, s, da, Kt, F, wp, D,
                     static_cast<float*>(dh));
  hipLaunchKernelGGL(gbwd_dw1_f32_kernel, dim3((unsigned)((n_red + 255) / 256)), blk, 0, s, da, hp, ld, Kt, F, D, zds,
                     ds, dW1, db1, dw2, db2);
  return hipGetLastError();
}

}  // namespace tg

// Gate MLP score of every token (TokenGate article, section "How does
// TokenGate learned token pruning work?": an MLP scores each token from its
// post-attention residual at the gate layer):
//     s_t = b2 + sum_f w2[f] * SiLU(b1[f] + W1[f, :] . hidden[t, :])
//
// bf16 path: one workgroup of 2 * F/64 waves scores 256 tokens.  The product
// is computed transposed, C^T[f][t] = W1[f] . h[t], with the 32x32x16 bf16
// MFMA, so that each lane of the accumulator holds one token's column and a
// run of F rows: the SiLU . w2 epilogue then reduces over F inside the lane,
// across the two wave halves, and across the F-quarter waves through LDS, in
// a fixed order (bit-reproducible, no atomics).  The [T, F] activation never
// reaches memory.  hidden and W1 stream through two LDS stages of 64
// columns: the next stage's global loads are issued before the current
// stage's MFMAs and written to LDS after them.
#include "tg_common.h"

namespace tg {
namespace {

constexpr int kGateBM = 256;  // tokens per workgroup
constexpr int kGateBK = 64;   // reduction columns per LDS stage
constexpr int kRowChunks = kGateBK / 8;  // 16-byte chunks per staged row
constexpr int kRowPad = kRowChunks + 1;  // padded row: 9 x 16 B, so 16
                                         // consecutive rows hit 16 bank groups
constexpr int kBufFlags = 0x00020000;    // raw buffer: reads past num_records give 0

template <int NFQ>  // number of 64-wide F quarters (F = 64 * NFQ)
__global__ __launch_bounds__(128 * NFQ) void gate_bf16_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld, int64_t T, int D,
    const uint16_t* __restrict__ W1, const float* __restrict__ b1,
    const float* __restrict__ w2, float b2, float* __restrict__ scores) {
  constexpr int F = 64 * NFQ;
  constexpr int NT = 128 * NFQ;                    // threads
  constexpr int H_CHUNKS = kGateBM * kRowChunks;   // 2048 chunks of hidden
  constexpr int W_CHUNKS = F * kRowChunks;
  constexpr int H_PER_T = H_CHUNKS / NT;
  constexpr int W_PER_T = W_CHUNKS / NT;
  static_assert(H_CHUNKS % NT == 0 && W_CHUNKS % NT == 0, "tile split");

  // Two LDS stages: the next 64 columns are written while these are read.
  __shared__ uint4 sh_h[2][kGateBM * kRowPad];
  __shared__ uint4 sh_w[2][F * kRowPad];
  __shared__ float sh_red[NFQ][kGateBM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / NFQ;  // token half: tokens [128 wt, 128 wt + 128)
  const int wf = wave % NFQ;  // F quarter: rows [64 wf, 64 wf + 64)
  const int64_t t0 = (int64_t)blockIdx.x * kGateBM;
  const int rows = (int)min((int64_t)kGateBM, T - t0);

  // hidden rows past T read as zero through the buffer descriptor; W1 is
  // always in range.
  int h_off[H_PER_T];
#pragma unroll
  for (int j = 0; j < H_PER_T; ++j) {
    const int id = tid + j * NT;
    h_off[j] = ((id / kRowChunks) * (int)ld + (id % kRowChunks) * 8) * 2;
  }
  int w_off[W_PER_T];
#pragma unroll
  for (int j = 0; j < W_PER_T; ++j) {
    const int id = tid + j * NT;
    w_off[j] = ((id / kRowChunks) * D + (id % kRowChunks) * 8) * 2;
  }
  uint4 pre_h[H_PER_T];
  uint4 pre_w[W_PER_T];
  const uint16_t* hbase = hidden + t0 * ld;

  // Global -> registers for reduction columns [k0, k0 + 64).
#define TG_GATE_PREFETCH(k0_)                                                                  \
  do {                                                                                         \
    const int k0 = (k0_);                                                                      \
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(                       \
        (void*)(hbase + k0), (short)0, rows * (int)ld * 2 - k0 * 2, kBufFlags);                \
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(                       \
        (void*)(W1 + k0), (short)0, F * D * 2 - k0 * 2, kBufFlags);                            \
    _Pragma("unroll") for (int j = 0; j < H_PER_T; ++j) pre_h[j] =                             \
        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, h_off[j], 0, 0));  \
    _Pragma("unroll") for (int j = 0; j < W_PER_T; ++j) pre_w[j] =                             \
        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[j], 0, 0));  \
  } while (0)
  // Registers -> LDS stage buf_.
#define TG_GATE_STAGE(buf_)                                                                    \
  do {                                                                                         \
    _Pragma("unroll") for (int j = 0; j < H_PER_T; ++j) {                                      \
      const int id = tid + j * NT;                                                             \
      sh_h[buf_][(id / kRowChunks) * kRowPad + (id % kRowChunks)] = pre_h[j];                  \
    }                                                                                          \
    _Pragma("unroll") for (int j = 0; j < W_PER_T; ++j) {                                      \
      const int id = tid + j * NT;                                                             \
      sh_w[buf_][(id / kRowChunks) * kRowPad + (id % kRowChunks)] = pre_w[j];                  \
    }                                                                                          \
  } while (0)

  f32x16 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  const int nk = D / kGateBK;
  TG_GATE_PREFETCH(0);
  TG_GATE_STAGE(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) TG_GATE_PREFETCH((kc + 1) * kGateBK);
#pragma unroll
    for (int ks = 0; ks < kGateBK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
      bf16x8 fa[2], fb[4];
#pragma unroll
      for (int fbk = 0; fbk < 2; ++fbk)
        fa[fbk] = as_bf16x8(sh_w[buf][(wf * 64 + fbk * 32 + (lane & 31)) * kRowPad + c]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        fb[tb] = as_bf16x8(sh_h[buf][(wt * 128 + tb * 32 + (lane & 31)) * kRowPad + c]);
#pragma unroll
      for (int fbk = 0; fbk < 2; ++fbk)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) acc[fbk][tb] = mfma32x32x16(fa[fbk], fb[tb], acc[fbk][tb]);
    }
    if (kc + 1 < nk) TG_GATE_STAGE(buf ^ 1);
    __syncthreads();
  }
#undef TG_GATE_PREFETCH
#undef TG_GATE_STAGE

  // Epilogue: lane holds token column (lane & 31) of each token block and F
  // rows acc_row(i, lane) of each F block.
  float bb[2][16], ww[2][16];
#pragma unroll
  for (int fbk = 0; fbk < 2; ++fbk)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int f = wf * 64 + fbk * 32 + acc_row(i, lane);
      bb[fbk][i] = b1 ? b1[f] : 0.0f;
      ww[fbk][i] = w2[f];
    }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float part = 0.0f;
#pragma unroll
    for (int fbk = 0; fbk < 2; ++fbk)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float a = acc[fbk][tb][i] + bb[fbk][i];
        const float z = a / (1.0f + __expf(-a));
        part = fmaf(ww[fbk][i], z, part);
      }
    part = pair_sum(part);
    if (lane < 32) sh_red[wf][wt * 128 + tb * 32 + lane] = part;
  }
  __syncthreads();
  for (int r = tid; r < kGateBM; r += NT) {
    const int64_t t = t0 + r;
    if (t < T) {
      float sum = 0.0f;
#pragma unroll
      for (int q = 0; q < NFQ; ++q) sum += sh_red[q][r];
      scores[t] = sum + b2;
    }
  }
}

// fp32 path: one wave per token, lanes split F; the dot products over D run
// sequentially in fp32, the F reduction is a fixed shuffle tree.
__global__ __launch_bounds__(256) void gate_f32_kernel(
    const float* __restrict__ hidden, int64_t ld, int64_t T, int D,
    const float* __restrict__ W1, const float* __restrict__ b1,
    const float* __restrict__ w2, float b2, int F, float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* h = hidden + t * ld;
  float part = 0.0f;
  for (int f = lane; f < F; f += 64) {
    const float* w = W1 + (int64_t)f * D;
    float a = b1 ? b1[f] : 0.0f;
    for (int k = 0; k < D; ++k) a = fmaf(w[k], h[k], a);
    const float z = a / (1.0f + __expf(-a));
    part = fmaf(w2[f], z, part);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
  if (lane == 0) scores[t] = part + b2;
}

}  // namespace

hipError_t launch_gate_bf16(const void* hidden, int64_t ld, int64_t T, int D, const void* W1,
                            const float* b1, const float* w2, float b2, int F, float* scores,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + kGateBM - 1) / kGateBM));
  const auto* h = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint16_t*>(W1);
  switch (F) {
    case 64: hipLaunchKernelGGL(gate_bf16_kernel<1>, grid, dim3(128), 0, s, h, ld, T, D, w, b1, w2, b2, scores); break;
    case 128: hipLaunchKernelGGL(gate_bf16_kernel<2>, grid, dim3(256), 0, s, h, ld, T, D, w, b1, w2, b2, scores); break;
    case 256: hipLaunchKernelGGL(gate_bf16_kernel<4>, grid, dim3(512), 0, s, h, ld, T, D, w, b1, w2, b2, scores); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gate_f32(const float* hidden, int64_t ld, int64_t T, int D, const float* W1,
                           const float* b1, const float* w2, float b2, int F, float* scores,
                           hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4));
  hipLaunchKernelGGL(gate_f32_kernel, grid, dim3(256), 0, s, hidden, ld, T, D, W1, b1, w2, b2, F,
                     scores);
  return hipGetLastError();
}

}  // namespace tg

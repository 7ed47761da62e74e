// Gate MLP score of every token (TokenGate article, section "How does
// TokenGate learned token pruning work?": an MLP scores each token from its
// post-attention residual at the gate layer):
//     s_t = b2 + sum_f w2[f] * SiLU(b1[f] + W1[f, :] . hidden[t, :])
//
// bf16 path: the product is computed transposed, C^T[f][t] = W1[f] . h[t],
// with the 32x32x16 bf16 MFMA.  A workgroup of 8 waves owns tiles of
// 256 / FS tokens: each wave owns 32 tokens and F / FS rows of W1 (FS = 1
// when the tokens fill every CU with 256-token tiles, 2 or 4 for shorter
// inputs), so that every lane of the accumulators holds one token's column.
// The SiLU . w2 epilogue reduces over F inside the lane, across the two wave
// halves and, for FS > 1, across the FS waves of a token group through LDS,
// in a fixed order (bit-reproducible, no atomics); the [T, F] activation
// never reaches memory.  hidden is read once, from HBM straight into the registers that
// serve as the MFMA's B operand, three stages of 64 columns ahead of their
// use (the register file holds far more bytes in flight than LDS could);
// W1, which every tile reads in full, streams through four LDS stages filled
// by buffer-to-LDS loads.  One workgroup per CU loops over tiles, and the
// loads run ahead across tile boundaries.
#include <atomic>

#include "tg_common.h"

namespace tg {
namespace {

constexpr int kGateBK = 64;    // reduction columns per stage (128-byte row segments)
constexpr int kGateAhead = 3;  // stages loaded ahead of the one computed
constexpr int kBufFlags = 0x00020000;  // raw buffer: reads past num_records give 0

// A staged row of W1 is 64 columns = eight 16-byte chunks; logical chunk c
// of row r sits at position c ^ ((r >> 1) & 7), so that the fragment reads
// of 16 consecutive rows at one chunk touch 16 different 16-byte bank groups.
__device__ __forceinline__ int gate_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// One 16-byte buffer-to-LDS load per lane: lane l writes bytes
// [16 l, 16 l + 16) of lds.  Out-of-range reads write zeros.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// Reduction order inside a stage.  A lane of half h = lane / 32 supplies,
// for k-step j, the 8 columns [32 h + 8 j, 32 h + 8 j + 8) of its stage: for
// hidden that is the j-th 16 bytes of the 64 contiguous bytes it loads, and
// the W1 fragments follow the same column map, so the products sum over the
// same columns as the definition, in another order.
// TAIL: D % 64 != 0 (a partial last stage; a separate instantiation, so the
// loads of full-width inputs carry no selects).
template <int NFB, int FS, bool TAIL>  // F = 32 * NFB, split over FS waves per token group
__global__ __launch_bounds__(512, 1) void gate_bf16_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld, int64_t T, int D, int n_tiles,
    const uint16_t* __restrict__ W1, const float* __restrict__ b1,
    const float* __restrict__ w2, float b2, float* __restrict__ scores) {
  constexpr int F = 32 * NFB;
  constexpr int NW = 8;
  constexpr int BM = 32 * NW / FS;    // tokens per tile
  constexpr int NFW = NFB / FS;       // F blocks per wave
  static_assert(NFB % FS == 0, "F split");
  constexpr int W_BYTES = F * kGateBK * 2;    // one stage of W1
  constexpr int W_DMA = W_BYTES / 1024 / NW;  // 1 KB buffer-to-LDS copies per wave per stage
  constexpr int PER = W_DMA + 4;              // vector-memory instructions per wave per stage
  static_assert(W_BYTES % (1024 * NW) == 0, "stage split");

  __shared__ __attribute__((aligned(16))) char sw0[W_BYTES], sw1[W_BYTES], sw2[W_BYTES], sw3[W_BYTES];
  __shared__ __attribute__((aligned(16))) float sb1[F], sw2v[F];
  __shared__ float sred[FS][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tgrp = wave / FS;  // token group: tokens [32 tgrp, 32 tgrp + 32) of the tile
  const int fpart = wave % FS; // F blocks [NFW fpart, NFW fpart + NFW)
  for (int f = tid; f < F; f += NW * 64) {
    sb1[f] = b1 ? b1[f] : 0.0f;
    sw2v[f] = w2[f];
  }

  // Stages per tile, rounded up to a multiple of four (the unroll below);
  // stages past D load zeros and add nothing.  With D % 64 != 0 the last
  // stage that holds columns of D (stage D / 64) is partial: there the
  // 16-byte chunks of both operands at or past column D (D % 8 == 0, so a
  // chunk is wholly in or out) are loaded from the first offset past the
  // buffer's range, which reads zeros, instead of from the next row.
  const int nk = ((D + kGateBK - 1) / kGateBK + 3) & ~3;
  const int tail_stage = (D % kGateBK) ? D / kGateBK : -1;
  const int tail_cols = D % kGateBK;
  const int my_tiles = ((int)blockIdx.x < n_tiles) ? (n_tiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int n_steps = my_tiles * nk;

  // hidden: lane loads 64 contiguous bytes of token tgrp * 32 + lane % 32:
  // chunk j holds columns 32 (lane / 32) + 8 j .. +7 of the stage
  const int h_voff = ((tgrp * 32 + (lane & 31)) * (int)ld + (lane >> 5) * 32) * 2;
  bool h_dead[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) h_dead[j] = 32 * (lane >> 5) + 8 * j >= tail_cols;
  // W1 copies: copy j of this wave fills rows 8 (wave * W_DMA + j) .. +7;
  // lane l writes position l % 8 of row l / 8, which holds that row's
  // logical chunk gate_swz(row, l % 8).
  int w_src[W_DMA];
  bool w_dead[W_DMA];  // the chunk lies past D in the partial stage
#pragma unroll
  for (int j = 0; j < W_DMA; ++j) {
    const int r = (wave * W_DMA + j) * 8 + (lane >> 3);
    const int c = gate_swz(r, lane & 7);  // logical chunk: columns 8 c .. 8 c + 7
    w_src[j] = (r * D + c * 8) * 2;
    w_dead[j] = 8 * c >= tail_cols;
  }
  // W1 fragment of F block fb, k-step ks: row 32 fb + lane % 32, logical
  // chunk 4 (lane / 32) + ks; the swizzle term depends on the lane only.
  int a_off[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    a_off[ks] = (fpart * NFW * 32 + (lane & 31)) * (kGateBK * 2) + gate_swz(lane & 31, 4 * (lane >> 5) + ks) * 16;

  // Load position: tile ld_tile (a multiple of gridDim.x past blockIdx.x),
  // stage ld_k of it.  Loads past the last tile read nothing (zero range).
  int ld_tile = blockIdx.x, ld_k = 0;
  auto issue = [&](char* sw, uint4 (&h)[4]) __attribute__((always_inline)) {
    const int64_t tt0 = (int64_t)ld_tile * BM;
    const int rows = ld_tile < n_tiles ? (int)min((int64_t)BM, T - tt0) : 0;
    const int k0 = ld_k * kGateBK;
    const bool kin = k0 < D;
    const int kk = kin ? k0 : 0;
    const int hb = __builtin_amdgcn_readfirstlane((rows > 0 && kin) ? rows * (int)ld * 2 - kk * 2 : 0);
    const int wb = __builtin_amdgcn_readfirstlane(kin ? F * D * 2 - kk * 2 : 0);
    const uint16_t* hb_ptr = rows > 0 ? hidden + tt0 * ld + kk : hidden;
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc((void*)hb_ptr, (short)0, hb, kBufFlags);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)(W1 + kk), (short)0, wb, kBufFlags);
    const bool tail = TAIL && ld_k == tail_stage;  // uniform
#pragma unroll
    for (int j = 0; j < W_DMA; ++j)
      lds_load16(rw, sw + (wave * W_DMA + j) * 1024, (tail && w_dead[j]) ? wb : w_src[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      h[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          rh, (tail && h_dead[j]) ? hb : h_voff + 16 * j, 0, 0));
    if (++ld_k == nk) {
      ld_k = 0;
      ld_tile += gridDim.x;
    }
  };

  f32x16 acc[NFW];
#pragma unroll
  for (int fb = 0; fb < NFW; ++fb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[fb][i] = 0.0f;

  // One stage: 4 k-steps x NFW F blocks; each W1 fragment is read three
  // MFMAs ahead of its use.
  constexpr int NM = 4 * NFW;
  constexpr int AHEAD = 3;
  auto compute = [&](const char* sw, const uint4 (&h)[4]) __attribute__((always_inline)) {
    bf16x8 fa[NM];
    auto frag = [&](int m) __attribute__((always_inline)) {
      const int ks = m / NFW, fb = m % NFW;
      return *reinterpret_cast<const bf16x8*>(sw + a_off[ks] + fb * 32 * (kGateBK * 2));
    };
#pragma unroll
    for (int m = 0; m < AHEAD; ++m) fa[m] = frag(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + AHEAD < NM) fa[m + AHEAD] = frag(m + AHEAD);
      __builtin_amdgcn_sched_barrier(0);
      const int ks = m / NFW, fb = m % NFW;
      acc[fb] = mfma32x32x16(fa[m], as_bf16x8(h[ks]), acc[fb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue of one tile: lane holds token column lane % 32 and F rows
  // 32 (NFW fpart + fb) + acc_row(i, lane).  With FS > 1 the partial sums of
  // a token group's waves meet in LDS and its first wave adds them in order.
  int ep_tile = blockIdx.x;
  auto epilogue = [&]() __attribute__((always_inline)) {
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int fb = 0; fb < NFW; ++fb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int f = (fpart * NFW + fb) * 32 + 8 * i4 + 4 * (lane >> 5);
        const float4 bb = *reinterpret_cast<const float4*>(&sb1[f]);
        const float4 ww = *reinterpret_cast<const float4*>(&sw2v[f]);
        const float bv[4] = {bb.x, bb.y, bb.z, bb.w}, wv[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float a = acc[fb][4 * i4 + c] + bv[c];
          const float z = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
          p[c] = fmaf(wv[c], z, p[c]);
        }
      }
    const float part = pair_sum((p[0] + p[1]) + (p[2] + p[3]));
    const int64_t t = (int64_t)ep_tile * BM + tgrp * 32 + lane;
    if (FS == 1) {
      if (lane < 32 && t < T) scores[t] = part + b2;
    } else {
      if (lane < 32) sred[fpart][tgrp * 32 + lane] = part;
      // LDS-only barrier: the loads in flight stay in flight.  sred is
      // written again only a tile later, many barriers on.
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (fpart == 0 && lane < 32 && t < T) {
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < FS; ++q) sum += sred[q][tgrp * 32 + lane];
        scores[t] = sum + b2;
      }
    }
    ep_tile += gridDim.x;
  };

  // End of a stage's wait: this wave's loads of the stage about to be
  // computed are complete (PER loads per stage, completing in order; the
  // two newer stages stay in flight) and its LDS reads of the previous
  // stage are done; then all waves meet, so the stage's W1 copy is whole and
  // the buffer the next loads fill is no longer read.
#define TG_GATE_SYNC() asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((kGateAhead - 1) * PER) : "memory")

  uint4 h0[4], h1[4], h2[4], h3[4];
  issue(sw0, h0);
  issue(sw1, h1);
  issue(sw2, h2);
  int kc = 0;
  for (int s = 0; s < n_steps; s += 4) {
    TG_GATE_SYNC();
    issue(sw3, h3);
    compute(sw0, h0);
    TG_GATE_SYNC();
    issue(sw0, h0);
    compute(sw1, h1);
    TG_GATE_SYNC();
    issue(sw1, h1);
    compute(sw2, h2);
    TG_GATE_SYNC();
    issue(sw2, h2);
    compute(sw3, h3);
    kc += 4;
    if (kc == nk) {
      kc = 0;
      epilogue();
#pragma unroll
      for (int fb = 0; fb < NFW; ++fb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[fb][i] = 0.0f;
    }
  }
#undef TG_GATE_SYNC
  // the loads issued past the last stage must land before the workgroup's
  // LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

hipError_t device_cu_count(int* n) {
  // queried once per device (concurrent first calls store the same value)
  static std::atomic<int> cu_count[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int c = cu_count[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    c = c > 0 ? c : 1;
    cu_count[dev].store(c, std::memory_order_relaxed);
  }
  *n = c;
  return hipSuccess;
}

hipError_t launch_gate_bf16(const void* hidden, int64_t ld, int64_t T, int D, const void* W1,
                            const float* b1, const float* w2, float b2, int F, float* scores,
                            hipStream_t s) {
  if (T == 0) return hipSuccess;
  // one workgroup per CU, each looping over tiles
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  // F split: the smallest that gives every CU a tile (256 / FS tokens each)
  const int nfb = F / 32;
  int fs = 1;
  while (fs < 4 && fs * 2 <= nfb && (T + 256 / fs - 1) / (256 / fs) < n_cu) fs *= 2;
  const int bm = 256 / fs;
  const int n_tiles = (int)((T + bm - 1) / bm);
  const dim3 grid((unsigned)min(n_tiles, n_cu));
  const auto* h = static_cast<const uint16_t*>(hidden);
  const auto* w = static_cast<const uint16_t*>(W1);
#define TG_GATE_LAUNCH(NFB_, FS_)                                                                                  \
  do {                                                                                                             \
    if (D % 64)                                                                                                    \
      hipLaunchKernelGGL((gate_bf16_kernel<NFB_, FS_, true>), grid, dim3(512), 0, s, h, ld, T, D, n_tiles, w, b1,  \
                         w2, b2, scores);                                                                          \
    else                                                                                                           \
      hipLaunchKernelGGL((gate_bf16_kernel<NFB_, FS_, false>), grid, dim3(512), 0, s, h, ld, T, D, n_tiles, w, b1, \
                         w2, b2, scores);                                                                          \
  } while (0)
  if (F == 64) {
    if (fs == 1) TG_GATE_LAUNCH(2, 1); else TG_GATE_LAUNCH(2, 2);
  } else if (F == 128) {
    if (fs == 1) TG_GATE_LAUNCH(4, 1); else if (fs == 2) TG_GATE_LAUNCH(4, 2); else TG_GATE_LAUNCH(4, 4);
  } else if (F == 256) {
    if (fs == 1) TG_GATE_LAUNCH(8, 1); else if (fs == 2) TG_GATE_LAUNCH(8, 2); else TG_GATE_LAUNCH(8, 4);
  } else {
    return hipErrorInvalidValue;
  }
#undef TG_GATE_LAUNCH
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

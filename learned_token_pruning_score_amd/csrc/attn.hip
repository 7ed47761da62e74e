// Token-gated causal GQA attention over the kept tokens (TokenGate article,
// section "What is token-gated attention?": each kept token's score becomes
// an additive bias on the attention logits above the gate, with a learnable
// per-head gain and a learnable temperature):
//     x_ij = tau * q_i . k_j / sqrt(d) + g_h * s_j,   j <= i within a prompt
//     o_i  = softmax_j(x_ij) v_j,  lse_i = ln sum_j exp(x_ij)
//
// bf16 path (gfx950 MFMA, fp32 accumulation): one workgroup of 8 waves per
// (query head, prompt, 256-row query tile); each wave owns 32 query rows.
// Short inputs (fewer 256-row tiles than twice the CUs) take the key-split
// schedule described at attn_bf16_ks_kernel instead.
//  * Scores are formed transposed, S^T = K Q^T, with the 32x32x16 MFMA: lane
//    l then holds 32 keys of query row (l & 31) per 64-key tile, so the
//    softmax max and sum are lane-local plus one exchange with lane l ^ 32.
//  * The bias and temperature fold into the score: the score accumulators
//    start at the key's bias c_j = g_h log2e s_j / scale (the MFMA's C
//    operand, read from LDS), so the accumulator holds q.k + c_j, the logit
//    is scale * acc, and p = exp2(scale * acc - scale * m) is one FMA and
//    one exp2 per score.
//  * P^T stays in registers: the accumulator layout of S^T is exactly the B
//    operand layout of O^T += V^T P^T once keys are relabelled (within each
//    16-key MFMA step, lane half G holds keys 4G..4G+3 and 8+4G..8+4G+3); V
//    stays row-major in LDS and a transposing LDS read delivers those keys.
//  * MFMA and vector ALU work overlap only across the waves of a SIMD, so
//    the two waves sharing a SIMD alternate: while one issues only MFMAs
//    (value product of its previous tile, scores of its next tile) the
//    other runs only the softmax of its current tile (see the schedule).
//  * Three LDS stages with padded rows (conflict-free fragment reads); the
//    K and V halves of each tile are loaded by the two wave groups in their
//    vector-ALU phases, one tile ahead.
//  * Causal masking only on the tile that crosses a wave's diagonal; tiles
//    are launched longest-first (tile index is the slowest grid dimension,
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
constexpr float kRescale = 8.0f;  // lazy-rescale threshold on the running max (log2 units)
// Fourth word of a raw buffer descriptor (32-bit data format, no swizzle):
// accesses at or past num_records read as zero.
constexpr int kBufFlags = 0x00020000;
constexpr int KAHEAD = 2;  // k-steps of K fragments read ahead of their MFMAs
constexpr int VAHEAD = 3;  // V fragments read ahead of their MFMAs

// One output row (query row l % 32 of the wave) from the O^T accumulators
// (block db holds head dimensions 32 db ..), scaled by inv, rounded to bf16
// and stored at op (the row's first head dimension) with 16-byte stores
// (store_row32_bf16); only `store` lanes write.
template <int NDB>
__device__ __forceinline__ void store_o_row(const f32x16 (&o)[NDB], float inv, int G, bool store, uint16_t* op) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    store_row32_bf16(op + 32 * db, G, store, [&](int i) __attribute__((always_inline)) { return o[db][i] * inv; });
}

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(
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
  constexpr int K_ITEMS = kBK * KCH;  // 16-byte chunks of a K (or V) tile
  // LDS rows are padded so that fragment reads spread over the banks: a K
  // row is HD*2 + 16 bytes (an odd number of 16-byte units), a V row HD*2 +
  // 64 bytes, so the eight rows one transposing read touches cover every
  // bank exactly twice.
  constexpr int KROW = KCH + 1;     // 16-byte units per padded K row
  constexpr int VROW = KCH + 4;     // 16-byte units per padded V row
  // Three LDS stages (see the schedule below).
  __shared__ uint4 sK[3][kBK * KROW];
  __shared__ uint4 sV[3][kBK * VROW];
  __shared__ __attribute__((aligned(16))) float sB[3][kBK];  // per key: g_h log2e s_j / scale

  const int x = blockIdx.x;
  const int h = head_swizzle ? (x % 8) * (Hq / 8) + x / 8 : x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  int b = 0, tile = n_qtiles - 1 - (int)blockIdx.z;
  if (gridDim.y > 1) {
    work_item(cu, (int)gridDim.y, n_qtiles, BQ, (long long)blockIdx.y + (long long)gridDim.y * blockIdx.z, lane, b, tile);
    b = __builtin_amdgcn_readfirstlane(b);
    tile = __builtin_amdgcn_readfirstlane(tile);
    if (tile < 0) return;
  }
  const int lo = cu[b];
  const int n = cu[b + 1] - lo;
  const int q0 = tile * BQ;
  if (q0 >= n) return;
  const int kvh = h / group;
  const int G = lane >> 5;
  // Waves w and w + 4 share a SIMD (the dispatcher places the waves of a
  // workgroup round-robin over the four SIMDs; another placement would only
  // cost speed).  They own the two 32-row halves of one 64-row block, so
  // both cross the causal diagonal in the same key tile.
  const int grp = wave >> 2;  // 0: first half of the block, 1: second
  const int qw = q0 + 64 * (wave & 3) + 32 * grp;
  const int my_q = qw + (lane & 31);
  // The key bias is the initial value of the score accumulators: the stage
  // holds c_j = g_h log2e s_j / scale per key in fp32 (0 without a bias), so
  // the accumulator holds q.k + c_j and the logit is scale * acc.  The
  // softmax then needs one FMA per score.  Requires scale > 0 (checked on
  // the host).
  const bool has_bias = (bias != nullptr) && (gain != nullptr);
  const float cmul = has_bias ? gain[h] * kLog2e / qk_scale : 0.0f;
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

  const float* bias_p = bias ? bias + lo : nullptr;

  // Staging split between the two wave groups, each in its vector ALU
  // phase: group 0 writes the K rows and the bias of a tile, group 1 its V
  // rows, 4 * 64 threads with HALF_T 16-byte chunks each.  Buffer-resource
  // loads: the descriptor of each tile starts at its first key and ends at
  // the prompt's last key (or 64 keys on), so rows past the prompt read as
  // zero without a branch, and a tile wholly past the prompt reads nothing.
  // Rows past the prompt only occur in a tile that crosses the causal
  // diagonal of every wave reading it, where they are masked.
  constexpr int HALF_T = K_ITEMS / (NT / 2);
  static_assert(K_ITEMS % (NT / 2) == 0, "half split");
  const int gtid = tid & (NT / 2 - 1);
  int h_off[HALF_T];
#pragma unroll
  for (int j = 0; j < HALF_T; ++j) {
    const int id = gtid + j * (NT / 2);
    h_off[j] = ((id / KCH) * (int)(grp == 0 ? ks : vs) + (id % KCH) * 8) * 2;
  }
  uint4 hreg[HALF_T], hreg1[HALF_T];
  float breg = 0.0f, breg1 = 0.0f;
  auto load_into = [&](int k0, uint4 (&hr)[HALF_T], float& br) __attribute__((always_inline)) {
    // wave-uniform (kept in scalar registers, so the descriptors are too)
    const int rows = __builtin_amdgcn_readfirstlane(max(min(n - k0, kBK), 0));
    const uint16_t* base = grp == 0 ? kbase + (int64_t)k0 * ks : vbase + (int64_t)k0 * vs;
    const int stride = grp == 0 ? (int)ks : (int)vs;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)base, (short)0, rows * stride * 2, kBufFlags);
#pragma unroll
    for (int j = 0; j < HALF_T; ++j)
      hr[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, h_off[j], 0, 0));
    if (grp == 0 && bias_p != nullptr) {
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(bias_p + k0), (short)0, rows * 4, kBufFlags);
      br = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (gtid & (kBK - 1)) * 4, 0, 0));
    }
  };
  auto prefetch_half = [&](int k0) __attribute__((always_inline)) { load_into(k0, hreg, breg); };
  auto stage_from = [&](int buf, const uint4 (&hr)[HALF_T], float br) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < HALF_T; ++j) {
      const int id = gtid + j * (NT / 2);
      if (grp == 0) sK[buf][(id / KCH) * KROW + (id % KCH)] = hr[j];
      else sV[buf][(id / KCH) * VROW + (id % KCH)] = hr[j];
    }
    if (grp == 0 && gtid < kBK) sB[buf][gtid] = has_bias ? br * cmul : 0.0f;
  };
  auto stage_half = [&](int buf) __attribute__((always_inline)) { stage_from(buf, hreg, breg); };

  // Scores S^T = K Q^T + bias of one tile into s, two interleaved MFMA
  // chains; the K fragments are read KAHEAD k-steps ahead.
  f32x16 s[2];
  auto qk = [&](int buf) __attribute__((always_inline)) {
    // The lane's address in the stage is made opaque once, so each
    // fragment read is that address plus an immediate offset.  kfrag: the
    // fragments of k-step st for both key halves.
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const u32x4 lds_u4;
    uint32_t ka = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)
        reinterpret_cast<const char*>(&sK[buf][(lane & 31) * KROW + G]);
    asm volatile("" : "+v"(ka));
    auto kfrag = [&](int st, uint4 (&f)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        f[kb] = __builtin_bit_cast(uint4, *(lds_u4*)(uintptr_t)(ka + ((kb * 32) * KROW + 2 * st) * 16));
    };
    // accumulators start at the key bias: register i of key half kb holds
    // key kb * 32 + 8 (i / 4) + 4 G + i % 4 (four consecutive keys per
    // 16-byte read, the same for a whole lane half)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 c = *reinterpret_cast<const float4*>(&sB[buf][kb * 32 + 8 * a + 4 * G]);
        s[kb][4 * a + 0] = c.x;
        s[kb][4 * a + 1] = c.y;
        s[kb][4 * a + 2] = c.z;
        s[kb][4 * a + 3] = c.w;
      }
    // each fragment has its own registers: no copies between steps
    uint4 f[NKS][2];
#pragma unroll
    for (int j = 0; j < KAHEAD; ++j) kfrag(j, f[j]);
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
      if (st + KAHEAD < NKS) kfrag(st + KAHEAD, f[st + KAHEAD]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(as_bf16x8(f[st][kb]), qf[st], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Softmax of the tile in s: masked max (MASK: the tile crosses the
  // wave's diagonal), lazy rescale of O (the running max only moves when a
  // row's max grows by more than kRescale, log2 units: until then
  // p <= 2^kRescale, harmless in fp32 and bf16), p = exp2(scale * acc -
  // scale * m), fp32 row sum, bf16 P^T.  P^T needs no shuffle: the S^T
  // accumulator layout equals the B-operand layout once keys are relabelled
  // (within each 16-key step, lane half G holds keys 4G..4G+3 and
  // 8+4G..8+4G+3), which is the order pv reads V^T in.
  bf16x8 pb[2][2];
  auto softmax = [&](int k0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
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
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[kb][hh][j] = (__bf16)s[kb][8 * hh + j];
    // the whole softmax stays in this (vector ALU) interval: nothing of it
    // may sink past the barrier into the wave's next (MFMA) interval
    __builtin_amdgcn_sched_barrier(0);
  };
  // O^T += V^T P^T for the tile whose probabilities are in pb, V^T
  // fragments read VAHEAD MFMAs ahead.  A transposing LDS read
  // (ds_read_b64_tr_b16) turns the row-major V tile into the MFMA operand:
  // within each 16-lane group, lane i receives element i % 4 of the 8-byte
  // chunks addressed by lanes 4j + i / 4 (j = 0..3).  Lane s of group g
  // therefore addresses key row 4 (g / 2) + s / 4 and columns
  // 16 (g % 2) + 4 (s % 4) .. +3 of a 16-key step, and lane l receives keys
  // 4G..4G+3 (then +8..+11) of head-dim row l % 32 of the block.
  auto pv = [&](int buf) __attribute__((always_inline)) {
    const int gi = lane & 15, g = lane >> 4;
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    uint32_t va = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(
        reinterpret_cast<const char*>(&sV[buf][0]) + (4 * (g >> 1) + (gi >> 2)) * (VROW * 16) +
        (16 * (g & 1) + 4 * (gi & 3)) * 2);
    asm volatile("" : "+v"(va));  // opaque lane address: reads use immediate offsets
    constexpr int NM = 4 * NDB;
    // fragment m = (kh, db): keys 32 (kh / 2) + 16 (kh % 2) .., head-dim block db
    auto vfrag = [&](int mi) __attribute__((always_inline)) {
      const int kh = mi / NDB, db = mi % NDB;
      const uint32_t a0 = va + ((kh >> 1) * 32 + 16 * (kh & 1)) * (VROW * 16) + db * 64;
      const s4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(uintptr_t)a0);
      const s4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(uintptr_t)(a0 + 8 * (VROW * 16)));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // each fragment has its own registers: no copies between steps
    bf16x8 vf[NM];
#pragma unroll
    for (int j = 0; j < VAHEAD; ++j) vf[j] = vfrag(j);
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      if (mi + VAHEAD < NM) vf[mi + VAHEAD] = vfrag(mi + VAHEAD);
      __builtin_amdgcn_sched_barrier(0);
      const int kh = mi / NDB, db = mi % NDB;
      o[db] = mfma32x32x16(vf[mi], pb[kh >> 1][kh & 1], o[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Schedule.  Each key tile takes two barrier intervals.  In every
  // interval one wave of each SIMD pair runs only MFMAs (the value product
  // of its previous tile, then the scores of its next tile) while the other
  // runs only vector ALU work (the softmax of its current tile, and its
  // group's share of the staging), so the matrix core and the vector ALU of
  // the SIMD are busy at the same time:
  //   interval 2t:     group 0: PV(t - 1), QK(t)    group 1: softmax(t - 1), V rows of t + 1
  //   interval 2t + 1: group 0: softmax(t), K rows of t + 1    group 1: PV(t - 1), QK(t)
  // Tile t sits in LDS stage t % 3: the K rows of tile t + 1 replace those
  // of tile t - 2 (last read in interval 2t - 3), its V rows those of tile
  // t - 2 (last read in interval 2t - 1).  Every wave takes part in every
  // barrier; the tile crossing its diagonal is its last and the only
  // masked one.
  const int t_diag = n_kt_w - 1;  // -1: no rows
  const int n_loop = n_kt + 1;    // the last value products come one tile late
  // unsigned, so the compiler knows LDS addresses are non-negative and folds
  // the per-fragment offsets into the instructions
  auto buf_of = [&](int t) __attribute__((always_inline)) { return (int)((unsigned)t % 3u); };
  // this group's half of tile t from the registers into its stage, then
  // the global loads of its half of tile t + 1 (landing two intervals on)
  auto stage_next = [&](int t) __attribute__((always_inline)) {
    stage_half(buf_of(t));
    prefetch_half((t + 1) * kBK);
  };
  // tile 1, loaded with tile 0 into registers of its own
  auto stage_first = [&]() __attribute__((always_inline)) {
    stage_from(buf_of(1), hreg1, breg1);
    prefetch_half(2 * kBK);
  };
  prefetch_half(0);
  load_into(kBK, hreg1, breg1);
  stage_half(0);
  __syncthreads();
  int t = 0;
  if (grp == 0) {
    if (t_diag >= 0) {
      qk(0);
      __syncthreads();
      stage_first();
      if (t_diag == 0) softmax(0, std::true_type{});
      else softmax(0, std::false_type{});
      __syncthreads();
      t = 1;
      for (; t < t_diag; ++t) {
        pv(buf_of(t - 1));
        qk(buf_of(t));
        __syncthreads();
        stage_next(t + 1);
        softmax(t * kBK, std::false_type{});
        __syncthreads();
      }
      if (t == t_diag) {
        pv(buf_of(t - 1));
        qk(buf_of(t));
        __syncthreads();
        stage_next(t + 1);
        softmax(t * kBK, std::true_type{});
        __syncthreads();
        ++t;
      }
      pv(buf_of(t - 1));  // t == t_diag + 1: the last value product
      __syncthreads();
      stage_next(t + 1);
      __syncthreads();
      ++t;
    }
    for (; t < n_loop; ++t) {
      __syncthreads();
      if (t == 0) stage_first();
      else stage_next(t + 1);
      __syncthreads();
    }
  } else {
    if (t_diag >= 0) {
      stage_first();
      __syncthreads();
      qk(0);
      __syncthreads();
      t = 1;
      for (; t <= t_diag; ++t) {
        stage_next(t + 1);
        softmax((t - 1) * kBK, std::false_type{});
        __syncthreads();
        pv(buf_of(t - 1));
        qk(buf_of(t));
        __syncthreads();
      }
      stage_next(t + 1);  // t == t_diag + 1
      softmax(t_diag * kBK, std::true_type{});
      __syncthreads();
      pv(buf_of(t - 1));
      __syncthreads();
      ++t;
    }
    for (; t < n_loop; ++t) {
      if (t == 0) stage_first();
      else stage_next(t + 1);
      __syncthreads();
      __syncthreads();
    }
  }

  if (!wave_active) return;
  const float l_tot = pair_sum(l_run);
  const int q_row = min(my_q, n - 1);  // rows past the prompt store nothing
  store_o_row(o, 1.0f / l_tot, G, my_q < n, out + (int64_t)(lo + q_row) * ((int64_t)Hq * HD) + (int64_t)h * HD);
  if (lse != nullptr && G == 0 && my_q < n)
    lse[(int64_t)h * Kt + lo + my_q] = (m_run * qk_scale + __log2f(l_tot)) * kLn2;
}

// Key-split schedule (short inputs, where the query tile that sees every
// key sets the kernel's time): one workgroup of 8 waves per (query head,
// prompt, 128-row query tile).  Waves w and w + 4 share a SIMD and own the
// same 32 query rows; wave w takes the even key tiles and wave w + 4 the odd
// ones, each keeping its own running max, row sum and O.  In interval i the
// group that owns tile i issues only MFMAs (the value product of its tile
// i - 2, then the scores of tile i) while the other group runs the softmax
// of tile i - 1, so one key tile is consumed per interval and the longest
// row takes half the intervals of the 256-row schedule.  Each group stages
// its own tiles: the K rows (and bias) of tile t + 2 are loaded in its
// MFMA interval t and written to LDS in its next (softmax) interval, the V
// rows of tile t + 2 loaded then and written in its MFMA interval t + 2,
// so one set of staging registers serves both.  K of tile t lives in LDS
// stage t % 2 (read in interval t), V of tile t in stage t % 3 (read in
// interval t + 2).  At the end the odd-tile waves hand (max, sum, O) to
// their partners through LDS, which merge them in a fixed order.
template <int HD>
__global__ __launch_bounds__(512, 1) void attn_bf16_ks_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t qs, int64_t ks, int64_t vs,
    const float* __restrict__ bias, const float* __restrict__ gain, float qk_scale,
    const int32_t* __restrict__ cu, int Hq, int group, int head_swizzle, int n_qtiles,
    int64_t Kt, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = 512;
  constexpr int BQ = 128;           // query rows per workgroup
  constexpr int KCH = HD / 8;
  constexpr int NKS = HD / 16;
  constexpr int NDB = HD / 32;
  constexpr int K_ITEMS = kBK * KCH;
  constexpr int KROW = KCH + 1;
  constexpr int VROW = KCH + 4;
  constexpr int K_STAGE = kBK * KROW;  // uint4 units
  constexpr int V_STAGE = kBK * VROW;
  constexpr int B_OFF = 2 * K_STAGE + 3 * V_STAGE;
  constexpr int LDS_U4 = B_OFF + (2 * kBK * 4) / 16;
  // the end-of-kernel merge reuses the same memory
  static_assert(4 * NDB * 16 * 64 + 2 * 4 * 64 <= 4 * B_OFF, "merge area");
  __shared__ uint4 smem[LDS_U4];
  float* const sB = reinterpret_cast<float*>(smem + B_OFF);  // [2][kBK]: g_h log2e s_j / scale

  const int x = blockIdx.x;
  const int h = head_swizzle ? (x % 8) * (Hq / 8) + x / 8 : x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int b = 0, tile = n_qtiles - 1 - (int)blockIdx.z;
  if (gridDim.y > 1) {
    work_item(cu, (int)gridDim.y, n_qtiles, BQ, (long long)blockIdx.y + (long long)gridDim.y * blockIdx.z, lane, b, tile);
    b = __builtin_amdgcn_readfirstlane(b);
    tile = __builtin_amdgcn_readfirstlane(tile);
    if (tile < 0) return;
  }
  const int lo = cu[b];
  const int n = cu[b + 1] - lo;
  const int q0 = tile * BQ;
  if (q0 >= n) return;
  const int kvh = h / group;
  const int G = lane >> 5;
  const int grp = wave >> 2;   // 0: even key tiles, 1: odd key tiles
  const int pair = wave & 3;
  const int qw = q0 + 32 * pair;
  const int my_q = qw + (lane & 31);
  const bool has_bias = (bias != nullptr) && (gain != nullptr);
  const float cmul = has_bias ? gain[h] * kLog2e / qk_scale : 0.0f;
  const float rs_thr = kRescale / qk_scale;

  bf16x8 qf[NKS];
  {
    const uint16_t* qp = q + (int64_t)(lo + my_q) * qs + (int64_t)h * HD + 8 * G;
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (my_q < n) u = *reinterpret_cast<const uint4*>(qp + 16 * st);
      qf[st] = as_bf16x8(u);
    }
  }
  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m_run = -INFINITY;
  float nms = 0.0f;
  float l_run = 0.0f;

  const int kv_end = min(q0 + BQ, n);
  const int n_kt = (kv_end + kBK - 1) / kBK;
  const bool wave_active = qw < n;
  const int t_diag = wave_active ? min(qw + 31, n - 1) / kBK : -1;  // the wave's masked tile
  const uint16_t* kbase = k + (int64_t)lo * ks + (int64_t)kvh * HD;
  const uint16_t* vbase = v + (int64_t)lo * vs + (int64_t)kvh * HD;
  const float* bias_p = bias ? bias + lo : nullptr;

  // Staging by the group's 256 threads, HALF_T 16-byte chunks each; buffer
  // loads read rows past the prompt as zero (see the 256-row kernel).
  constexpr int HALF_T = K_ITEMS / (NT / 2);
  static_assert(K_ITEMS % (NT / 2) == 0, "half split");
  const int gtid = tid & (NT / 2 - 1);
  int k_off[HALF_T], v_off[HALF_T];
#pragma unroll
  for (int j = 0; j < HALF_T; ++j) {
    const int id = gtid + j * (NT / 2);
    k_off[j] = ((id / KCH) * (int)ks + (id % KCH) * 8) * 2;
    v_off[j] = ((id / KCH) * (int)vs + (id % KCH) * 8) * 2;
  }
  uint4 hreg[HALF_T];
  float breg = 0.0f;
  auto rows_of = [&](int t) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(max(min(n - t * kBK, kBK), 0));
  };
  auto load_k = [&](int t) __attribute__((always_inline)) {
    const int rows = rows_of(t);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kbase + (int64_t)t * kBK * ks), (short)0, rows * (int)ks * 2, kBufFlags);
#pragma unroll
    for (int j = 0; j < HALF_T; ++j)
      hreg[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, k_off[j], 0, 0));
    if (bias_p != nullptr) {
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(bias_p + t * kBK), (short)0, rows * 4, kBufFlags);
      breg = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (gtid & (kBK - 1)) * 4, 0, 0));
    }
  };
  auto load_v = [&](int t) __attribute__((always_inline)) {
    const int rows = rows_of(t);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vbase + (int64_t)t * kBK * vs), (short)0, rows * (int)vs * 2, kBufFlags);
#pragma unroll
    for (int j = 0; j < HALF_T; ++j)
      hreg[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, v_off[j], 0, 0));
  };
  auto kbuf = [&](int t) __attribute__((always_inline)) { return (int)((unsigned)t & 1u); };
  auto vbuf = [&](int t) __attribute__((always_inline)) { return (int)((unsigned)t % 3u); };
  auto store_k = [&](int t) __attribute__((always_inline)) {
    uint4* sk = smem + kbuf(t) * K_STAGE;
#pragma unroll
    for (int j = 0; j < HALF_T; ++j) {
      const int id = gtid + j * (NT / 2);
      sk[(id / KCH) * KROW + (id % KCH)] = hreg[j];
    }
    if (gtid < kBK) sB[kbuf(t) * kBK + gtid] = has_bias ? breg * cmul : 0.0f;
  };
  auto store_v = [&](int t) __attribute__((always_inline)) {
    uint4* sv = smem + 2 * K_STAGE + vbuf(t) * V_STAGE;
#pragma unroll
    for (int j = 0; j < HALF_T; ++j) {
      const int id = gtid + j * (NT / 2);
      sv[(id / KCH) * VROW + (id % KCH)] = hreg[j];
    }
  };

  f32x16 s[2];
  auto qk = [&](int t) __attribute__((always_inline)) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const u32x4 lds_u4;
    const int kb_ = kbuf(t);
    uint32_t ka = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)
        reinterpret_cast<const char*>(smem + kb_ * K_STAGE + (lane & 31) * KROW + G);
    asm volatile("" : "+v"(ka));
    auto kfrag = [&](int st, uint4 (&f)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        f[kb] = __builtin_bit_cast(uint4, *(lds_u4*)(uintptr_t)(ka + ((kb * 32) * KROW + 2 * st) * 16));
    };
    // accumulators start at the key bias (see the 256-row kernel)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 c = *reinterpret_cast<const float4*>(&sB[kb_ * kBK + kb * 32 + 8 * a + 4 * G]);
        s[kb][4 * a + 0] = c.x;
        s[kb][4 * a + 1] = c.y;
        s[kb][4 * a + 2] = c.z;
        s[kb][4 * a + 3] = c.w;
      }
    uint4 f[NKS][2];
#pragma unroll
    for (int j = 0; j < KAHEAD; ++j) kfrag(j, f[j]);
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
      if (st + KAHEAD < NKS) kfrag(st + KAHEAD, f[st + KAHEAD]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(as_bf16x8(f[st][kb]), qf[st], s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  bf16x8 pb[2][2];
  auto softmax = [&](int k0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
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
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][i], qk_scale, nms));
        psum += s[kb][i];
      }
    l_run += psum;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[kb][hh][j] = (__bf16)s[kb][8 * hh + j];
    // the whole softmax stays in this (vector ALU) interval: nothing of it
    // may sink past the barrier into the wave's next (MFMA) interval
    __builtin_amdgcn_sched_barrier(0);
  };
  auto pv = [&](int t) __attribute__((always_inline)) {
    const int gi = lane & 15, g = lane >> 4;
    typedef short s4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4 lds_s4;
    uint32_t va = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(
        reinterpret_cast<const char*>(smem + 2 * K_STAGE + vbuf(t) * V_STAGE) +
        (4 * (g >> 1) + (gi >> 2)) * (VROW * 16) + (16 * (g & 1) + 4 * (gi & 3)) * 2);
    asm volatile("" : "+v"(va));
    constexpr int NM = 4 * NDB;
    auto vfrag = [&](int mi) __attribute__((always_inline)) {
      const int kh = mi / NDB, db = mi % NDB;
      const uint32_t a0 = va + ((kh >> 1) * 32 + 16 * (kh & 1)) * (VROW * 16) + db * 64;
      const s4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(uintptr_t)a0);
      const s4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(uintptr_t)(a0 + 8 * (VROW * 16)));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 vf[NM];
#pragma unroll
    for (int j = 0; j < VAHEAD; ++j) vf[j] = vfrag(j);
#pragma unroll
    for (int mi = 0; mi < NM; ++mi) {
      if (mi + VAHEAD < NM) vf[mi + VAHEAD] = vfrag(mi + VAHEAD);
      __builtin_amdgcn_sched_barrier(0);
      const int kh = mi / NDB, db = mi % NDB;
      o[db] = mfma32x32x16(vf[mi], pb[kh >> 1][kh & 1], o[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Schedule of group grp (its own tiles t = grp, grp + 2, ... up to the
  // wave's diagonal tile; interval i ends with the i-th barrier):
  //   interval t (MFMA):     V rows of t to LDS, load K of t + 2, PV(t - 2), QK(t)
  //   interval t + 1 (VALU): softmax(t), K of t + 2 to LDS, load V of t + 2
  // then one more MFMA interval for the last value product, and staging
  // only until every wave has passed n_int barriers.
  const int n_int = n_kt + 3;
  if (grp == 0) {
    load_k(0);
    store_k(0);
    load_v(0);
  } else {
    load_k(1);
  }
  __syncthreads();
  int i = 0;
  if (grp == 1) {  // interval 0 of the odd group: staging only
    store_k(1);
    load_v(1);
    __syncthreads();
    i = 1;
  }
  if (t_diag >= grp) {
    int t = grp;
    store_v(t);
    load_k(t + 2);
    qk(t);
    __syncthreads();
    if (t == t_diag) softmax(t * kBK, std::true_type{});
    else softmax(t * kBK, std::false_type{});
    store_k(t + 2);
    load_v(t + 2);
    __syncthreads();
    t += 2;
    for (; t < t_diag; t += 2) {
      store_v(t);
      load_k(t + 2);
      pv(t - 2);
      qk(t);
      __syncthreads();
      softmax(t * kBK, std::false_type{});
      store_k(t + 2);
      load_v(t + 2);
      __syncthreads();
    }
    if (t == t_diag) {
      store_v(t);
      load_k(t + 2);
      pv(t - 2);
      qk(t);
      __syncthreads();
      softmax(t * kBK, std::true_type{});
      store_k(t + 2);
      load_v(t + 2);
      __syncthreads();
      t += 2;
    }
    store_v(t);  // the last value product
    load_k(t + 2);
    pv(t - 2);
    __syncthreads();
    store_k(t + 2);
    load_v(t + 2);
    __syncthreads();
    i = t + 2;
  }
  for (; i < n_int; ++i) {
    if (((i ^ grp) & 1) == 0) {
      store_v(i);
      load_k(i + 2);
    } else {
      store_k(i + 1);
      load_v(i + 1);
    }
    __syncthreads();
  }

  // Merge: the odd-tile wave of each pair hands its partial state to the
  // even-tile wave through LDS (the stages are no longer read).  (Both waves
  // merging and each storing half of the head dimensions measured slower.)
  float* mO = reinterpret_cast<float*>(smem);  // [pair][db][i][lane]
  float* mM = mO + 4 * NDB * 16 * 64;          // [pair][lane]
  float* mL = mM + 4 * 64;
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) mO[((pair * NDB + db) * 16 + i2) * 64 + lane] = o[db][i2];
    mM[pair * 64 + lane] = m_run;
    mL[pair * 64 + lane] = l_run;
  }
  __syncthreads();
  if (grp == 1 || !wave_active) return;
  const float m1 = mM[pair * 64 + lane];
  const float l1 = mL[pair * 64 + lane];
  const float m_all = fmaxf(m_run, m1);  // finite: the diagonal tile is one group's
  const float a0 = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m_run - m_all) * qk_scale);
  const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((m1 - m_all) * qk_scale);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i2 = 0; i2 < 16; ++i2)
      o[db][i2] = o[db][i2] * a0 + mO[((pair * NDB + db) * 16 + i2) * 64 + lane] * a1;
  const float l_tot = pair_sum(l_run * a0 + l1 * a1);
  const int q_row = min(my_q, n - 1);  // rows past the prompt store nothing
  store_o_row(o, 1.0f / l_tot, G, my_q < n,
              out + (int64_t)(lo + q_row) * ((int64_t)Hq * HD) + (int64_t)h * HD);
  if (lse != nullptr && G == 0 && my_q < n)
    lse[(int64_t)h * Kt + lo + my_q] = (m_all * qk_scale + __log2f(l_tot)) * kLn2;
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
  // 8 waves (4 SIMD pairs), 32 query rows each
  constexpr int NW = 8;
  const int swz = (Hq % 8 == 0 && ((Hq / 8) % group) == 0) ? 1 : 0;
  const float qk_scale = tau * kLog2e / sqrtf((float)d);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(out);
  // Few 256-row query tiles (short inputs): the tile that sees every key
  // sets the time, and the key-split schedule halves its intervals.
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  if ((int64_t)Hq * ((Kt + 255) / 256) < 2 * (int64_t)n_cu) {
    const int n_qt = (max_len + 127) / 128;
    const dim3 g2((unsigned)Hq, (unsigned)B, (unsigned)n_qt);
    if (d == 128)
      hipLaunchKernelGGL((attn_bf16_ks_kernel<128>), g2, dim3(512), 0, s, qq, kk, vv, qs, ks, vs, bias,
                         gain, qk_scale, cu_kept, Hq, group, swz, n_qt, Kt, oo, lse);
    else if (d == 64)
      hipLaunchKernelGGL((attn_bf16_ks_kernel<64>), g2, dim3(512), 0, s, qq, kk, vv, qs, ks, vs, bias,
                         gain, qk_scale, cu_kept, Hq, group, swz, n_qt, Kt, oo, lse);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const int n_qtiles = (max_len + 32 * NW - 1) / (32 * NW);
  const dim3 grid((unsigned)Hq, (unsigned)B, (unsigned)n_qtiles);
  if (d == 128) {
    hipLaunchKernelGGL((attn_bf16_kernel<128, NW>), grid, dim3(64 * NW), 0, s, qq, kk, vv, qs, ks,
                       vs, bias, gain, qk_scale, cu_kept, Hq, group, swz, n_qtiles, Kt, oo, lse);
  } else if (d == 64) {
    hipLaunchKernelGGL((attn_bf16_kernel<64, NW>), grid, dim3(64 * NW), 0, s, qq, kk, vv, qs, ks,
                       vs, bias, gain, qk_scale, cu_kept, Hq, group, swz, n_qtiles, Kt, oo, lse);
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

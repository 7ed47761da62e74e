// Internal declarations shared by the HIP kernels and the C-ABI layer.
// Nothing here is part of the public ABI (include/tg.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32x16 bf16 MFMA (gfx950): D = A(32x16) * B(16x32) + C, fp32 accumulate.
// Operand layout used throughout: lane l holds A[l % 32][8 * (l / 32) + j] and
// B[8 * (l / 32) + j][l % 32] for j = 0..7; accumulator register i of lane l
// holds C[8 * (i / 4) + 4 * (l / 32) + (i % 4)][l % 32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// One row of a 32x32 accumulator block rounded to bf16 and stored at p[0..31]:
// lane l holds row l % 32 and, in register i, column 8 (i / 4) + 4 G + i % 4
// (G = l / 32); val(i) is the fp32 value of register i.  The two lane halves
// first swap 4-column runs (v_permlane32_swap), so that each lane holds 8
// consecutive columns and the row leaves in two 16-byte stores of one lane
// pair: half the store instructions of 8-byte stores, each carrying twice
// the bytes of a row (store instructions that touch 32 rows were measured
// to cost kernel time).  Every lane takes part in the swaps; only `store`
// lanes write.
template <typename Val>
__device__ __forceinline__ void store_row32_bf16(uint16_t* p, int G, bool store, Val val) {
  auto pack2 = [&](int i) __attribute__((always_inline)) {
    return (unsigned)__builtin_bit_cast(uint16_t, (__bf16)val(i)) |
           ((unsigned)__builtin_bit_cast(uint16_t, (__bf16)val(i + 1)) << 16);
  };
  uint4 w[2];
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    // u: columns 16 pp + 4 G .. +3 (registers 8 pp ..), v: 16 pp + 8 + 4 G .. +3
    unsigned u[2], v[2], x0[2], x1[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u[j] = pack2(8 * pp + 2 * j);
      v[j] = pack2(8 * pp + 4 + 2 * j);
      // lanes < 32 receive the upper half's u, lanes >= 32 the lower half's v
      const auto r = __builtin_amdgcn_permlane32_swap(u[j], v[j], false, false);
      x0[j] = r[0];
      x1[j] = r[1];
    }
    w[pp] = G == 0 ? make_uint4(u[0], u[1], x1[0], x1[1]) : make_uint4(x0[0], x0[1], v[0], v[1]);
  }
  if (!store) return;
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) *reinterpret_cast<uint4*>(p + 16 * pp + 8 * G) = w[pp];
}

// Work order of the tiled attention kernels with several prompts.  Their
// grid has a slot (y, z) for every prompt and every tile index up to the
// longest prompt's tile count, of rank r = y + B z in dispatch order (the
// head index x runs fastest), but prompt b has only n_b = ceil(len_b / BQ)
// tiles.  A slot whose tile does not exist exits at once; spread through the
// dispatch order, such slots were measured to hold back the dispatch of the
// real ones (about 176 of 256 CUs busy on a ragged batch).  So rank r takes
// the r-th existing (prompt, index) pair in the order index descending, then
// prompt ascending, and the ranks past the last pair take the empty slots.
// Every wave computes the same mapping (no barrier): S(t), the number of
// pairs with index >= t, is a sum over the prompts of max(0, n_b - t), and
// the pair's index is the largest t with S(t) > r.
__device__ __forceinline__ int tiles_of(const int32_t* cu, int b, int BQ) {
  return (cu[b + 1] - cu[b] + BQ - 1) / BQ;
}
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ void work_item(const int32_t* __restrict__ cu, int B, int n_qt, int BQ,
                                          long long r, int lane, int& b_out, int& t_out) {
  const int nb0 = lane < B ? tiles_of(cu, lane, BQ) : 0;  // the first 64 prompts, kept in a register
  auto S = [&](int t) -> long long {
    long long s = max(0, nb0 - t);
    for (int b0 = 64; b0 < B; b0 += 64)
      if (b0 + lane < B) s += max(0, tiles_of(cu, b0 + lane, BQ) - t);
    return wave_sum_ll(s);
  };
  t_out = -1;
  b_out = 0;
  if (S(0) <= r) return;  // past the last pair
  int lo = 0, hi = n_qt;   // S(lo) > r >= S(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (S(mid) > r) lo = mid;
    else hi = mid;
  }
  long long j = r - S(lo + 1);  // rank among the prompts that have tile lo
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int bb = b0 + lane;
    const int nb = b0 == 0 ? nb0 : (bb < B ? tiles_of(cu, bb, BQ) : 0);
    const bool has = bb < B && nb > lo;
    const unsigned long long m = __ballot(has);
    const int c = __popcll(m);
    if (j < c) {
      const int below = __popcll(m & ((1ull << lane) - 1ull));
      const unsigned long long hit = __ballot(has && below == (int)j);
      b_out = b0 + __ffsll((long long)hit) - 1;
      t_out = lo;
      return;
    }
    j -= c;
  }
}

// Row of the 32x32 accumulator that register i of lane l holds.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// v_permlane32_swap with both operands equal to x leaves, in every lane,
// x of that lane in one result and x of lane l ^ 32 in the other.  A
// symmetric combination of the two is therefore the pairwise reduction,
// evaluated in the same operand order in both halves of the wave.
__device__ __forceinline__ float pair_max(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Compute units of the current device (queried once per device).
hipError_t device_cu_count(int* n);

// ---------------------------------------------------------------- launchers
hipError_t launch_gate_bf16(const void* hidden, int64_t ld, int64_t T, int D, const void* W1,
                            const float* b1, const float* w2, float b2, int F, float* scores,
                            hipStream_t s);
hipError_t launch_gate_f32(const float* hidden, int64_t ld, int64_t T, int D, const float* W1,
                           const float* b1, const float* w2, float b2, int F, float* scores,
                           hipStream_t s);

size_t select_workspace_bytes(int B, int64_t T);
// Allocation-free selection: bytes of scratch a call needs (0 when the
// one-workgroup path runs), the capacity of the static scratch array, and
// its address on the current device.
size_t select_scratch_bytes_needed(int B, int64_t T);
size_t select_static_scratch_capacity();
hipError_t select_static_scratch(hipStream_t stream, void** ptr);
hipError_t launch_select(const float* scores, const int32_t* cu, const int32_t* db,
                         const int32_t* de, const int32_t* budget, int B, int64_t T,
                         uint8_t* keep, void* ws, hipStream_t s);

size_t compact_workspace_bytes(int B, int64_t T);
hipError_t launch_compact(const void* hidden, int64_t ld, int D, int elem_bytes, const int32_t* pos,
                          const float* scores, const uint8_t* keep, const int32_t* cu,
                          const int32_t* db, const int32_t* de, int B, int64_t T, int64_t Kt,
                          void* hidden_out, int32_t* pos_out, float* bias_out,
                          int32_t* kept_idx_out, void* ws, hipStream_t s);

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, int64_t qs, int64_t ks,
                            int64_t vs, const float* bias, const float* gain, float tau,
                            const int32_t* cu_kept, int B, int max_len, int64_t Kt, int Hq,
                            int Hkv, int d, void* out, float* lse, hipStream_t s);
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, int64_t qs, int64_t ks,
                           int64_t vs, const float* bias, const float* gain, float tau,
                           const int32_t* cu_kept, int B, int max_len, int64_t Kt, int Hq,
                           int Hkv, int d, float* out, float* lse, hipStream_t s);

hipError_t launch_rope_table(const int32_t* pos, int64_t n, int d, double theta, float* table,
                             hipStream_t s);
hipError_t launch_qkv_rope_bf16(const void* x, int64_t ld, int64_t Kt, int D, const void* W,
                                const float* rope, int Hq, int Hkv, int d, void* out,
                                int64_t ld_out, hipStream_t s);
size_t attn_bwd_workspace_bytes(int B, int64_t Kt, int Hq, int Hkv, int d, int elem_bytes, int max_len);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                           const float* bias, const float* gain, float tau, const int32_t* cu, int B,
                           int max_len, int64_t Kt, int Hq, int Hkv, int d, int elem_bytes, const void* out,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, float* ds,
                           float* dg, float* dtau, void* ws, hipStream_t s);
hipError_t launch_proj_store(const void* x, int64_t ld, int64_t n, int K, const void* W, int N, void* out,
                             int64_t ld_out, hipStream_t s);
size_t gate_bwd_workspace_bytes(int64_t Kt, int D, int F, int elem_bytes);
hipError_t launch_gate_bwd(const void* h, int64_t ld, int64_t Kt, int D, const void* W1, const float* b1,
                           const float* w2, int F, const float* dbias, const int32_t* kept_idx,
                           const int32_t* cu, const int32_t* db, const int32_t* de, int B, int elem_bytes,
                           void* dh, float* dW1, float* db1, float* dw2, float* db2, void* ws,
                           hipStream_t s);
size_t decode_workspace_bytes(int B, int Hq, int d, int max_len);
hipError_t launch_kv_scatter(const void* k, const void* v, int64_t sks, int64_t svs, const float* bias,
                             const int32_t* cu, int B, int64_t Kt, int Hkv, int d, int elem_bytes, void* kc,
                             void* vc, int64_t ks, int64_t vs, float* bc, const int32_t* start, hipStream_t s);
hipError_t launch_kv_append(const void* kn, const void* vn, int B, int Hkv, int d, int elem_bytes, void* kc, void* vc,
                            int64_t ks, int64_t vs, float* bc, const int32_t* start, const int32_t* pos, hipStream_t s);
hipError_t launch_decode_attn(const void* q, const void* kc, const void* vc, int64_t ks, int64_t vs, const float* bc,
                              const float* gain, float tau, const int32_t* start, const int32_t* lens, int B,
                              int max_len, int Hq, int Hkv, int d, int elem_bytes, void* out, float* lse, void* ws,
                              hipStream_t s);
hipError_t launch_rms_norm(const void* x, int64_t ld, int64_t n, int D, const float* w, float eps,
                           int elem_bytes, void* out, int64_t ld_out, hipStream_t s);
hipError_t launch_linear_residual(const void* a, int64_t ld, int64_t n, int K, const void* W, int N,
                                  const void* res, int64_t ld_res, int elem_bytes, void* out,
                                  int64_t ld_out, hipStream_t s);
hipError_t launch_swiglu(const void* h, int64_t ld, int64_t n, int K, const void* Wg, const void* Wu,
                         int I, int elem_bytes, void* out, int64_t ld_out, hipStream_t s);
hipError_t launch_qkv_rope_f32(const float* x, int64_t ld, int64_t Kt, int D, const float* W,
                               const float* rope, int Hq, int Hkv, int d, float* out,
                               int64_t ld_out, hipStream_t s);

}  // namespace tg

// skv_tile.h -- 16-key K/V tiles streamed into LDS by direct-to-LDS buffer
// loads, and the matrix-core helpers that read them (gfx950).  Shared by the
// split-K attention and the per-step score kernels.
//
// A tile holds 16 consecutive rows (keys) of K or V.  One direct-to-LDS copy
// moves 1 KB (64 lanes x 16 bytes) and lands contiguously, so copy u of a
// tile carries rows u, u + NI, u + 2 NI, ...; each lane fetches the 16-byte
// piece that belongs at its slot under the XOR swizzles below, which keeps
// the LDS reads of the MFMA operands free of bank conflicts.
#pragma once
#include "skv_common.h"
#include "skv_mfma.h"

namespace skv {
namespace {

constexpr int kStep = 16;  // keys per tile (one wave step)

#define SKV_LDS __attribute__((address_space(3)))
typedef short short4_t __attribute__((ext_vector_type(4)));

template <int D>
struct TileGeom {
  static constexpr int kRB = D * 2;              // bytes per bf16 row
  static constexpr int kPPR = kRB / 16;          // 16-byte pieces per row
  static constexpr int kRPI = 1024 / kRB;        // rows per direct-to-LDS copy (1 KB)
  static constexpr int kNI = kStep / kRPI;       // copies per tile (each of K and V)
  static constexpr int kTB = kStep * kRB;        // bytes per tile
  static constexpr int kKS = D / 32;             // k-steps of the q.K^T MFMA
  static constexpr int kNT = D / 16;             // 16-column tiles of the P.V MFMA
};

// Piece swizzles (XOR on the 16-byte piece index) of tile row t.  K rows are
// read 16 rows x one piece per 16 lanes; V is read transposed, 4 rows x two
// pieces per 16 lanes (8 rows per 32 lanes).  Both make those groups hit
// distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int t) {
  return D == 128 ? (t & 15) : ((((t >> 2) << 1) | (t & 1)) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int t) {
  return D == 128 ? 2 * (t & 7) : 2 * ((t & 1) | (((t >> 2) & 1) << 1));
}
// Staged query rows (row-major, D / 8 pieces per row): the 16 rows one MFMA
// operand read touches land on distinct banks.
template <int D>
__device__ __forceinline__ int swz_q(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// LDS byte of piece slot `pos` of tile row t: copy u = t % NI writes 1 KB
// holding rows u, u + NI, u + 2 NI, ...
template <int D>
__device__ __forceinline__ int tile_byte(int t, int pos) {
  using TG = TileGeom<D>;
  return (t % TG::kNI) * 1024 + (t / TG::kNI) * TG::kRB + pos * 16;
}

// s_waitcnt with vmcnt <= N and the other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Wait until at most min(newer, N) groups of PER copies are outstanding.
template <int N, int PER>
__device__ __forceinline__ void wait_newer(int newer) {
  if constexpr (N == 0) {
    wait_vm<0>();
  } else {
    if (newer >= N) wait_vm<N * PER>();
    else wait_newer<N - 1, PER>(newer);
  }
}

__device__ __forceinline__ floatx4_t mfma16(const short4_t& a, const short4_t& b, const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS: the wave's 64 pieces land
// contiguously (1 KB) at the wave-uniform LDS address `lds` (non-temporal).
__device__ __forceinline__ void copy_to_lds(BufRsrc r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SKV_LDS void*)lds, 16, voff, soff, 0, 2);
}
// Transposing LDS read: within each 16 lanes, lane j receives element j % 4 of
// the 8-byte pieces addressed by lanes 4k + j / 4, k = 0..3.
__device__ __forceinline__ short4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SKV_LDS short4_t*)p);
}

// Two floats to packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{x, y}, bf16x2_t));
}


}  // namespace
}  // namespace skv

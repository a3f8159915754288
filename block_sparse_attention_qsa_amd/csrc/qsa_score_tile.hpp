// a1 building block shared by the scoring kernels: the block scores of one
// 16-row compressed-key tile against up to 4 index queries on one bf16 MFMA
// 16x16x32 chain.
//
// The arex-research.com article (section on the four optimisations, item 2)
// lets up to 4 verify queries of a request share one load of each
// compressed-key tile; here the key rows are the M side of the MFMA and the
// queries the N side (4 of 16 columns used).  Products of two BF16 values are
// exact and accumulate in FP32.
//
// Step kk of the chain contracts dimensions 32kk .. 32kk+31: lane l = 16g + n
// of a wave takes bytes 64kk + 16g .. 64kk + 16g + 15 of key row n of the
// tile (from the wave's LDS copy of it, below) as its A operand.  The result
// leaves lane (g, n) with query n's scores of rows 4g .. 4g+3.
#pragma once

#include "qsa_common.hpp"

namespace qsa {

constexpr int kKeyRowBytes = QSA_INDEX_DIM * 2;

struct KeyTile {
  u32x4 w[4];    // step kk: dimensions 32kk + 8g .. 32kk + 8g + 7 of row n
};

// The request's index queries as the MFMA B operand: lane (g, n) holds query
// n's dimensions 32kk + 8g .. + 7 for step kk (zeros for n >= nq).
__device__ __forceinline__ void load_index_queries(bf16x8 (&qb)[4], const uint16_t* idx_q, int qs, int nq, int n,
                                                   int g) {
  const bool valid = n < nq;
  // The load always reads a real row (query qs for the unused columns) and is
  // masked afterwards: no branch, so all four loads issue back to back.
  const uint16_t* qp = idx_q + (int64_t)(qs + (valid ? n : 0)) * QSA_INDEX_DIM + 8 * g;
  const uint32_t keep = valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qb[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 32 * kk) & keep);
}

// Key tile staged in LDS (4 KiB per wave) by direct-to-LDS loads.  Load
// instruction i moves rows 4i .. 4i+3: lane l fetches 16-byte chunk
// (l mod 16) XOR row of row 4i + l/16 and the hardware stores it at byte 16l
// of that instruction's 1 KiB, so LDS slot s of row r holds chunk s XOR r.
// Each aligned group of 8 lanes fetches one whole 128-byte line (the XOR
// only permutes chunks within a line or swaps a row's two lines), so every
// instruction reads 1 KiB of whole lines and can stream past the caches
// (non-temporal).  Reading back, lane (g, n) takes chunk 4kk + g of row n
// from slot (4kk + g) XOR n: the 16 lanes of one g hit 16 different bank
// groups.
constexpr int kTileBytes = 16 * kKeyRowBytes;
constexpr int kCpolStream = 2;                 // non-temporal

__device__ __forceinline__ void load_key_tile_lds(uint8_t* tile_lds, __amdgpu_buffer_rsrc_t rs, int row0, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);
    const int chunk = (lane & 15) ^ row;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(tile_lds + 1024 * i), 16,
        (row0 + row) * kKeyRowBytes + 16 * chunk, 0, 0, kCpolStream);
  }
}

__device__ __forceinline__ void read_key_tile_lds(KeyTile& t, const uint8_t* tile_lds, int n, int g) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    t.w[kk] = *reinterpret_cast<const u32x4*>(tile_lds + kKeyRowBytes * n + 16 * ((4 * kk + g) ^ n));
}

__device__ __forceinline__ f32x4 contract_key_tile(const KeyTile& t, const bf16x8 (&qb)[4]) {
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.w[kk]), qb[kk], acc, 0, 0, 0);
  return acc;
}

}  // namespace qsa

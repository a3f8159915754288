// The step before block scoring: compressed index keys of the blocks that the
// tokens appended since the previous step have completed.
//
// The arex-research.com article (section on the four optimisations, item 1)
// groups tokens into 4-token micro-blocks and computes one compressed index
// key per block; it does not state the compression.  The key used here is the
// mean of the block's four per-token index keys, summed in FP64 in token order
// and rounded once to BF16 (nearest, ties to even).  Four BF16 values whose
// exponents differ by at most 43 need at most 53 significand bits in their
// sum, so the FP64 sum is then exact and the result the correctly rounded
// mean.
//
// One workgroup per request; each wave takes one new block at a time, lane l
// owning dimensions 2l and 2l+1 (one 4-byte load per token, 256 B per wave).
#include "qsa_common.hpp"
#include "qsa_launch.hpp"

namespace qsa {

// Round a double to BF16 bits, nearest with ties to even, saturating to
// infinity past the largest finite BF16 value.
__device__ __forceinline__ uint32_t bf16_rne_from_f64(double x) {
  const uint32_t sign = (__double_as_longlong(x) < 0) ? 0x8000u : 0u;
  if (x != x) return 0x7FC0u | sign;
  const double a = fabs(x);
  // halfway between the largest finite BF16, (2 - 2^-7) * 2^127, and 2^128
  if (a >= 3.3961775292304957e38) return 0x7F80u | sign;
  int e;
  (void)frexp(a, &e);                         // a = f * 2^e, f in [0.5, 1)
  const int qe = max(e - 1, -126) - 7;        // exponent of one BF16 unit in the last place at a
  const double quantum = ldexp(1.0, qe);
  const double r = rint(a / quantum) * quantum;   // a / quantum is exact; rint rounds half to even
  return (__float_as_uint((float)r) >> 16) | sign;   // r is a BF16 value, so the float is exact
}

__global__ __launch_bounds__(256) void compress_keys_kernel(Meta m, const int32_t* __restrict__ prev_len,
                                                            const uint32_t* __restrict__ tok_keys,
                                                            uint32_t* __restrict__ ckeys) {
  const int r = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int L1 = m.seq_len[r];
  int L0 = prev_len[r];
  if (threadIdx.x == 0) QSA_DCHECK(m.err, L0 >= 0 && L0 <= L1, QSA_ERROR_BAD_QUERIES);
  L0 = L0 < 0 ? 0 : (L0 > L1 ? L1 : L0);
  const int b_end = L1 >> 2;                  // blocks with 4b + 3 < L1
  const int b_first = L0 >> 2;                // blocks with 4b + 3 >= L0
  const int64_t row0 = m.blk_start[r];
  constexpr int kWords = QSA_INDEX_DIM / 2;   // 32-bit words (2 BF16) per key row
  for (int b = b_first + wave; b < b_end; b += nwaves) {
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t] = tok_keys[(int64_t)token_slot(m, r, 4 * b + t) * kWords + lane];
    double lo = (double)__uint_as_float(w[0] << 16), hi = (double)__uint_as_float(w[0] & 0xFFFF0000u);
#pragma unroll
    for (int t = 1; t < 4; ++t) {
      lo += (double)__uint_as_float(w[t] << 16);
      hi += (double)__uint_as_float(w[t] & 0xFFFF0000u);
    }
    ckeys[(row0 + b) * kWords + lane] = bf16_rne_from_f64(lo * 0.25) | (bf16_rne_from_f64(hi * 0.25) << 16);
  }
}

hipError_t launch_compress_keys(const Meta& m, const int32_t* prev_len, const void* tok_keys, void* ckeys,
                                hipStream_t stream) {
  compress_keys_kernel<<<m.num_req, 256, 0, stream>>>(m, prev_len, static_cast<const uint32_t*>(tok_keys),
                                                      static_cast<uint32_t*>(ckeys));
  return hipGetLastError();
}

}  // namespace qsa

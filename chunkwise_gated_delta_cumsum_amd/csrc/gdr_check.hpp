// Input range check (gdr_check_inputs): one streaming pass over the inputs
// that records, as bits of one device word, whether they break the numeric
// preconditions of the 16-bit path (see the numerics notes in gdr.h).
//
// * Non-finite values in q, k, v, g or beta (fp32, bf16 or fp16 encodings).
// * bf16 q, k or v whose magnitude rounds to infinity in fp16 (|x| >= 65520
//   rounds up past 65504; the largest bf16 below that is 65280, the
//   smallest above it 65536): the MFMA operands are fp16, and bf16 -> fp16
//   is exact for every value below.
// * Decays that grow within a chunk: the prep folds exp(sum of g over rows
//   of one chunk) into fp16 operands, which stay in range while the positive
//   g of one channel (or of the row decay) within any chunk sum to at most
//   kDecayLimit.  g <= 0 never sets the bit.
//
// Bits are set with one atomic OR per wave that found something; the word is
// cleared first by a one-lane kernel on the same stream.  The kernels are in
// gdr_launch_check.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr.h"

namespace gdr {

constexpr float kDecayLimit = 8.f;

typedef uint32_t chk_u32x4 __attribute__((ext_vector_type(4)));
typedef float chk_f32x4 __attribute__((ext_vector_type(4)));

struct CheckArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  uint32_t* flags;
  size_t nqk, nv, nbeta;  // elements of q (= of k), of v, of beta
  int B, T, HV, K, C, N;  // shapes; N = ceil(T / C) chunks per sequence
  bool perch;             // g is [B, T, HV, K] (else [B, T, HV])
  int fmt;                // q, k, v: 0 fp32, 1 bf16, 2 fp16
  bool qk_range;          // check q and k against the fp16 range (bf16 only)
  bool decay;             // check the positive g sums (the 16-bit path)
};

}  // namespace gdr

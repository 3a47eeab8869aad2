// The decode kernels for several queries per sequence (q_len * G <= 16
// (query, head) columns per wave; templates in decode_kernels.h).
//
// This translation unit is built with the MFMA accumulators in AGPRs (the
// compiler's default), not in VGPRs as the other kernels are.  Measured on
// MI355X: in the VGPR form these kernels gave results that varied from one
// call to the next on identical inputs, by a bf16 rounding step in up to
// half of the outputs (bf16 and fp32 KV, in every split mode), while the
// one-query and fp8 kernels built the same way repeated bit for bit; built
// with AGPR accumulators (and, for the balanced kernel, without the
// three-waves-per-SIMD hint that forces the VGPR form) every call repeats
// bit for bit, at the same speed (draft verification, 64 x 4 queries:
// balanced 116.5 against 118.1 us, one pass 118.8 against 118.4), and the
// balanced kernel then has room to stage its partials in LDS (112.8 us).
#include "decode_kernels.h"

namespace pa {

int launch_decode_mq(const DecodeArgs& a, void* stream) {
    return (int)dispatch<true>(a, LaunchF{a, reinterpret_cast<hipStream_t>(stream)});
}

int balanced_splits_mq(const DecodeArgs& a) { return dispatch<true>(a, SplitsF{a}); }

}  // namespace pa

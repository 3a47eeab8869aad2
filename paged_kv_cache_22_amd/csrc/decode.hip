// Decode entry points, and the kernels for one query per sequence (the
// templates are in decode_kernels.h; several queries per sequence are
// instantiated in decode_mq.hip, built with other code-generation flags).
#include "decode_kernels.h"

namespace pa {

int balanced_splits(const DecodeArgs& a) {
    return a.q_len > 1 ? balanced_splits_mq(a) : dispatch<false>(a, SplitsF{a});
}

int launch_decode(const DecodeArgs& a, void* stream) {
    if (a.num_seqs == 0) return 0;
    if (a.q_len > 1) return launch_decode_mq(a, stream);
    return (int)dispatch<false>(a, LaunchF{a, reinterpret_cast<hipStream_t>(stream)});
}

}  // namespace pa

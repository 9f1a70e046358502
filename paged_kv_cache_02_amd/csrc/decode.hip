// Paged decode for block sizes of 16 and more: instantiates the engine and
// the two schedules of decode_impl.h, and routes block size 8 to
// decode_bs8.hip.

#include "decode_impl.h"

namespace pkv {

int decode_heads_per_unit(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

pkv_status launch_decode_bf16(const DecodeArgs &a, hipStream_t stream)
{
    if (a.bs_log2 == 3) return launch_decode_bf16_bs8(a, stream);
    return launch_part_all<false>(a, stream);
}

pkv_status launch_decode_stream_bf16(const StreamArgs &a, hipStream_t stream)
{
    if (a.bs_log2 == 3) return launch_decode_stream_bf16_bs8(a, stream);
    return launch_stream_all<false>(a, stream);
}

}  // namespace pkv

// Paged decode for block size 8: the engine and schedules of decode_impl.h
// with each 16-token tile read from two blocks.

#include "decode_impl.h"

namespace pkv {

pkv_status launch_decode_bf16_bs8(const DecodeArgs &a, hipStream_t stream)
{
    return launch_part_all<true>(a, stream);
}

pkv_status launch_decode_stream_bf16_bs8(const StreamArgs &a, hipStream_t stream)
{
    return launch_stream_all<true>(a, stream);
}

}  // namespace pkv

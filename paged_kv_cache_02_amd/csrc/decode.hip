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

// One wave merges HU heads of one sequence, 16 bytes of each head row per
// lane (HU = 256 / D, fewer when the head count is not a multiple).
pkv_status launch_stream_merge(const StreamArgs &a, hipStream_t stream)
{
    int HU = 256 / a.D;
    while (a.Hq % HU) HU >>= 1;
    const long long grid = ((long long)a.B * (a.Hq / HU) + 3) / 4;
    if (grid <= 0) return PKV_OK;
    if (grid > 0x7fffffffLL) return PKV_ERR_SHAPE;
    const dim3 g((unsigned)grid), blk(256);
    if (a.D == 128) {
        if (HU == 2) hipLaunchKernelGGL((stream_merge_kernel<128, 2>), g, blk, 0, stream, a);
        else hipLaunchKernelGGL((stream_merge_kernel<128, 1>), g, blk, 0, stream, a);
    } else {
        if (HU == 4) hipLaunchKernelGGL((stream_merge_kernel<64, 4>), g, blk, 0, stream, a);
        else if (HU == 2) hipLaunchKernelGGL((stream_merge_kernel<64, 2>), g, blk, 0, stream, a);
        else hipLaunchKernelGGL((stream_merge_kernel<64, 1>), g, blk, 0, stream, a);
    }
    return launch_status();
}

pkv_status launch_decode_stream_bf16(const StreamArgs &a, hipStream_t stream)
{
    if (a.bs_log2 == 3) return launch_decode_stream_bf16_bs8(a, stream);
    return launch_stream_all<false>(a, stream);
}

}  // namespace pkv

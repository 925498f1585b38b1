// The plain form of the fused decode-step walk kernel (seq_walk.h): every
// (bit width, M) instantiation, and its entry-point table.
#include "seq_walk.h"

namespace mbq {

const void *seq_kernel_plain(int bits, int64_t M) {
#define MBQ_PICK(B, MM) return reinterpret_cast<const void *>(&seq_kernel<B, MM, false>)
    if (bits == 4) {
        switch (M) { case 1: MBQ_PICK(4, 1); case 2: MBQ_PICK(4, 2); case 3: MBQ_PICK(4, 3);
                     case 4: MBQ_PICK(4, 4); case 5: MBQ_PICK(4, 5); case 6: MBQ_PICK(4, 6);
                     case 7: MBQ_PICK(4, 7); default: MBQ_PICK(4, 8); }
    }
    switch (M) { case 1: MBQ_PICK(6, 1); case 2: MBQ_PICK(6, 2); case 3: MBQ_PICK(6, 3);
                 case 4: MBQ_PICK(6, 4); case 5: MBQ_PICK(6, 5); case 6: MBQ_PICK(6, 6);
                 case 7: MBQ_PICK(6, 7); default: MBQ_PICK(6, 8); }
#undef MBQ_PICK
}

hipError_t launch_sequence(int bits, int64_t M, bool full, int grid, int lds_bytes, const void *plan, uint32_t *err,
                           hipStream_t st) {
    void *args[] = {(void *)&plan, (void *)&err};
    const void *fn = full ? seq_kernel_full(bits, M) : seq_kernel_plain(bits, M);
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kSeqBlock), args, (unsigned)lds_bytes, st);
}

}  // namespace mbq

// ddh_sort.hip - the stable key/value radix sort of the map builder's cell
// sort, from the hipCUB library (rocPRIM backend). Kept in a translation unit
// of its own: the library's kernels are not part of the builder's code.
#include <hipcub/hipcub.hpp>

#include "ddh_internal.h"

namespace ddh {

int sort_pairs(void* temp, size_t* temp_bytes, const uint32_t* keys_in, uint32_t* keys_out,
               const int32_t* vals_in, int32_t* vals_out, int n, int end_bit, hipStream_t s)
{
    const hipError_t e = hipcub::DeviceRadixSort::SortPairs(temp, *temp_bytes, keys_in, keys_out,
                                                            vals_in, vals_out, n, 0, end_bit, s);
    if (e != hipSuccess)
        return hip_fail(e, "hipcub::DeviceRadixSort::SortPairs");
    return DDH_OK;
}

}  // namespace ddh

/*
 * hbm_copy.h -- C ABI of libhbm_copy.so, a plain 16-byte-vector device copy.
 *
 * It is the measuring stick for the RMSNorm kernels, not part of the RMSNorm
 * operation: the bandwidth a kernel that reads N bytes and writes N bytes can
 * reach on this GPU (the TileLang tutorial ch. 02, section 2.2, sets datasheet
 * against attainable bandwidth;
 * it notes that a copy mix reaches only part of the quoted HBM
 * bandwidth), and the known-size kernel used to scale the FETCH_SIZE and
 * WRITE_SIZE hardware counters into bytes.
 */
#ifndef MBR_HBM_COPY_H
#define MBR_HBM_COPY_H

#include <stdint.h>

#define HBM_COPY_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes from device pointer src to device pointer dst on `stream`
 * (hipStream_t, NULL = default), asynchronously.  Both pointers must be 16-byte
 * aligned and the ranges must not overlap.  max_blocks > 0 caps the grid
 * (grid-stride loop); 0 = one workgroup per 16 KiB of data.
 * Returns 0 on success, 1 on an invalid argument (nothing launched), 3 if the
 * launch failed.
 */
HBM_COPY_API int hbm_copy(const void* src, void* dst, int64_t bytes, int32_t max_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MBR_HBM_COPY_H */

// Internal: the thread-local last-error text behind pa_last_error() and the shape
// check of pa_decode, shared by every source file of the library.  Not part of the
// C ABI (hidden symbols).
#ifndef PA_STATUS_H_
#define PA_STATUS_H_

#include "pa.h"

namespace pa {

// Record a printf-style message as this thread's last error and return `st`.
__attribute__((visibility("hidden"), format(printf, 2, 3))) pa_status set_error(pa_status st,
                                                                               const char* fmt, ...);
// Clear this thread's last error and return PA_OK.
__attribute__((visibility("hidden"))) pa_status clear_error();
// PA_OK if pa_decode is built for this element type, head_dim and block_size; else
// PA_ERR_UNSUPPORTED with the last error set.
__attribute__((visibility("hidden"))) pa_status check_dtype_shape(pa_dtype dtype, int32_t head_dim,
                                                                  int32_t block_size);

}  // namespace pa

#endif  // PA_STATUS_H_

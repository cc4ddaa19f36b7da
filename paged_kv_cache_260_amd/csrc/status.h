// Status and error-message helpers shared by the C-ABI entry points.
#pragma once

namespace pkv {

// Records a printf-style message as this thread's last error and returns
// `status` (a pkv_status).
int set_error(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears this thread's last error and returns PKV_OK.
int clear_error();

}  // namespace pkv

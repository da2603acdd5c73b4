// Error reporting shared by the HIP and the host-only sources of libekh: sets
// the thread-local message that ekh_last_error() returns and passes the code
// through.
#pragma once

namespace ekh {
int report_error(int code, const char *msg);
} // namespace ekh

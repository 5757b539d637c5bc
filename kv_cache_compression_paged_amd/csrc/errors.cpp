// Error reporting of the C ABI: a thread-local message for the last failed
// call and the names of the status codes. Plain C++ (no GPU calls), shared by
// the library and by its host-only sanitizer build.
#include <cstdarg>
#include <cstdio>

#include "zipage.h"
#include "zp_host.h"

namespace zp {

namespace {
thread_local char g_msg[512] = "";
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
}

zp_status fail(zp_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

}  // namespace zp

extern "C" {

const char* zp_status_str(zp_status s) {
  switch (s) {
    case ZP_OK: return "ZP_OK";
    case ZP_EINVAL: return "ZP_EINVAL";
    case ZP_EUNSUPPORTED: return "ZP_EUNSUPPORTED";
    case ZP_EWORKSPACE: return "ZP_EWORKSPACE";
    case ZP_ENOSPACE: return "ZP_ENOSPACE";
    case ZP_EHIP: return "ZP_EHIP";
    case ZP_EDEVICE: return "ZP_EDEVICE";
    case ZP_ESYNC: return "ZP_ESYNC";
    default: return "ZP_UNKNOWN";
  }
}

const char* zp_last_error(void) { return zp::g_msg; }

}  // extern "C"

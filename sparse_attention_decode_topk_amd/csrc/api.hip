// Status strings and version of the C ABI.
#include "common.hpp"

extern "C" const char* dsa_status_str(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    default: return "DSA_ERR_UNKNOWN";
  }
}

extern "C" int dsa_version(void) { return 100; }

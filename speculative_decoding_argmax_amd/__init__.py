"""MI355X-native MTP draft / verify LM-head path.

The HIP library (``csrc/`` -> ``lib/libmtp.so``) is bound in ``mtp``; this
package's import does not load it, so the input generator (``workloads``)
works on machines without the built library.
"""

__all__ = ["workloads"]

"""MI355X-native GPT-2 training step: Python binding of the ``libtt`` C-ABI."""
